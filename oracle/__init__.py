"""TEST INFRASTRUCTURE: the float64 CPU oracle of the QSA select phase and the
checker that compares a device result with it.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never uses it, and it never uses the HIP
library: the two share nothing but the seeded input generators (qsa_inputs).

Arithmetic contract (Strata pull request #228, part 1, "arithmetic contract"
paragraph; Strata pull request #856, "Arithmetic contract and parity"):
    |s_gpu - score_ref| <= B = 2^-9.5 * S + 8 * 2^-24 * |score_ref|
with S the float64 sum of |k_b[i] * q_h[i]|.  A +2.5*B perturbation must fail
the same check (negative control, both pages).  Selected ids agree except at
near-ties whose gap is within 2*B (PR #856, "near-tie-gap guard").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

BOUND_REL = 2.0 ** -9.5
BOUND_ABS = 8.0 * 2.0 ** -24
NEG_CONTROL = 2.5
# Selection ids may differ from the oracle's only between blocks whose
# score_ref gap is within this many bounds (the larger of the two cells'
# B): the near-tie-gap guard of Strata pull request #856, "Arithmetic
# contract and parity", read as "gap <= 2*B".
NEAR_TIE_FACTOR = 2.0

_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_abi_version.restype = ctypes.c_int
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = None
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f32_to_f16_one.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16_one.restype = ctypes.c_uint16
        L.oracle_convert_f32_f16.argtypes = [_vp, _vp, _i64]
        L.oracle_convert_f32_f16.restype = None
        L.oracle_scores.argtypes = [_vp, ctypes.c_int, _i64, _vp, _i64, _i32, _i32, _i32, _i32,
                                    _i64, _vp, _i64, _vp, _vp, _vp, _i64]
        L.oracle_scores.restype = ctypes.c_int
        L.oracle_block_model_f32.argtypes = [_vp, _i64, _vp, _i64, _i32, _i32, _i32, _i32, _i64,
                                             _vp, _i64, _vp]
        L.oracle_block_model_f32.restype = ctypes.c_int
        L.oracle_topk.argtypes = [_vp, _i64, _i64, _i64, _i32, _vp, _i64, _vp]
        L.oracle_topk.restype = ctypes.c_int
        L.oracle_round_ratio_f16.argtypes = [_i64, _i64]
        L.oracle_round_ratio_f16.restype = ctypes.c_uint16
        L.oracle_block_keys.argtypes = [_vp, _i64, _i32, _i32, _i64, _i32, _vp, _i64]
        L.oracle_block_keys.restype = ctypes.c_int
        L.oracle_attention.argtypes = [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _i32, _i32, _i32,
                                       _i32, _i64, _i32, _i32, _vp, _vp]
        L.oracle_attention.restype = ctypes.c_int
        _lib = L
    return _lib


def max_threads() -> int:
    return lib().oracle_max_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's following parallel regions."""
    lib().oracle_set_threads(int(n))


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_vp)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.oracle_f16_to_f64(int(b)) for b in flat]).reshape(np.shape(bits))


def convert_f32_f16(x: np.ndarray) -> np.ndarray:
    src = np.ascontiguousarray(x, dtype=np.float32)
    dst = np.empty(src.shape, dtype=np.uint16)
    lib().oracle_convert_f32_f16(_p(src), _p(dst), src.size)
    return dst


@dataclass
class Scores:
    score: np.ndarray  # float64 [n_rows][nb]
    S: np.ndarray
    B: np.ndarray
    rows: np.ndarray   # int64 row ids r = g*nq + t


def scores(q: np.ndarray, kblk: np.ndarray, nb: int, rows: np.ndarray | None = None) -> Scores:
    """R1 of the oracle.  q is uint16 fp16 bits or float32 [nq][G][H][D];
    kblk is uint16 [G][>=nb][D].  rows: optional int64 list of g*nq + t."""
    q = np.ascontiguousarray(q)
    nq, G, H, D = q.shape
    kblk = np.ascontiguousarray(kblk, dtype=np.uint16)
    assert kblk.shape[0] == G and kblk.shape[2] == D and kblk.shape[1] >= nb
    if q.dtype == np.float32:
        is32 = 1
    else:
        assert q.dtype == np.uint16
        is32 = 0
    if rows is None:
        rows = np.arange(G * nq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.size
    ld = max(nb, 1)
    sc = np.empty((n, ld))
    S = np.empty((n, ld))
    B = np.empty((n, ld))
    rc = lib().oracle_scores(_p(q), is32, G * H * D, _p(kblk), kblk.shape[1] * D, G, nq, H, D, nb,
                             _p(rows), n, _p(sc), _p(S), _p(B), ld)
    assert rc == 0
    return Scores(sc[:, :nb], S[:, :nb], B[:, :nb], rows)


def block_model_f32(q16: np.ndarray, kblk: np.ndarray, b: int,
                    rows: np.ndarray | None = None, force_tail: bool = False) -> np.ndarray:
    """R2: fixed-order fp32 scores of block b for each requested row.  With
    force_tail the forced-tail rule follows the head sum: s = fl32(s + 1e9)."""
    q16 = np.ascontiguousarray(q16, dtype=np.uint16)
    nq, G, H, D = q16.shape
    kblk = np.ascontiguousarray(kblk, dtype=np.uint16)
    if rows is None:
        rows = np.arange(G * nq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty(rows.size, dtype=np.float32)
    rc = lib().oracle_block_model_f32(_p(q16), G * H * D, _p(kblk), kblk.shape[1] * D, G, nq, H,
                                      D, b, _p(rows), rows.size, _p(out))
    assert rc == 0
    if force_tail:
        out = (out + np.float32(FORCE_TAIL_ADD)).astype(np.float32)   # one IEEE fp32 addition
    return out


# The forced-tail rule.  Strata pull request #856 ("What") says the WMMA arm
# keeps the shared tail kernel's "+1e9 dead-tail rule" exactly, without
# defining it.  Reading taken: the partial last block (present when n_kv % bs
# != 0) gets 1e9 added to its score after the head sum, so that the block
# holding the newest tokens ranks first in every row's selection whatever its
# keys score.
FORCE_TAIL_ADD = 1e9


def force_tail(ref: Scores, n_kv: int, bs: int) -> Scores:
    """R1 followed by the forced-tail rule: the partial block's exact score
    plus 1e9 (float64), and that cell's bound recomputed from the contract
    for the new score, 2^-9.5*S + 8*2^-24*|score|.  Its second term grows by
    8*2^-24*1e9 (about 477), which covers the device's one fp32 rounding of
    s + 1e9 (at most half an ulp: 32 below 2^30, 64 below 2^31).  Without a
    partial block the scores are returned unchanged."""
    nf, nb = n_kv // bs, -(-n_kv // bs)
    if nb == nf:
        return ref
    score, B = ref.score.copy(), ref.B.copy()
    score[:, nf] = score[:, nf] + FORCE_TAIL_ADD
    B[:, nf] = 2.0 ** -9.5 * ref.S[:, nf] + 8.0 * 2.0 ** -24 * np.abs(score[:, nf])
    return Scores(score, ref.S, B, ref.rows)


def topk(score_rows: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """R3: ids [rows][k] (int32, -1 padded) and their scores (-inf padded)."""
    s = np.ascontiguousarray(score_rows, dtype=np.float64)
    if s.ndim == 1:
        s = s[None, :]
    rows, nb = s.shape
    ids = np.full((rows, k), -1, dtype=np.int32)
    vals = np.full((rows, k), -np.inf)
    if rows == 0 or k == 0 or nb == 0:
        return ids, vals
    rc = lib().oracle_topk(_p(s), nb, rows, nb, k, _p(ids), k, _p(vals))
    assert rc == 0
    return ids, vals


def round_ratio_f16(num: int, den: int) -> int:
    """fp16 bits nearest (ties to even) to num / den * 2^-24."""
    return int(lib().oracle_round_ratio_f16(int(num), int(den)))


def block_keys(k_tok: np.ndarray, n_kv: int, bs: int) -> np.ndarray:
    """The block key of every (KV head, block): the mean of the block's token
    keys rounded once to the nearest fp16 (the reading taken for k_b, which
    the pages index but do not define).  k_tok is uint16 fp16 bits
    [n_tok >= n_kv][G][D]; returns uint16 [G][nb][D]."""
    k = np.ascontiguousarray(k_tok, dtype=np.uint16)
    n_tok, G, D = k.shape
    assert n_tok >= n_kv
    nb = -(-n_kv // bs)
    out = np.zeros((G, max(nb, 1), D), dtype=np.uint16)
    rc = lib().oracle_block_keys(_p(k), G * D, G, D, n_kv, bs, _p(out), max(nb, 1) * D)
    assert rc == 0
    return out[:, :nb]


def attention(q16: np.ndarray, k_tok: np.ndarray, v_tok: np.ndarray, ids: np.ndarray,
              n_kv: int, bs: int) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of every query head over the tokens of the blocks
    its (KV head, query) row selected (the reading taken for the step after
    the selection), in float64, and the bound B of a fp32 device result.
    q16 uint16 [nq][G][H][D]; k_tok, v_tok uint16 [>= n_kv][G][D]; ids
    int32 [G][nq][k] (negative = empty slot).  Returns (out, B), float64
    [nq][G][H][D]."""
    q = np.ascontiguousarray(q16, dtype=np.uint16)
    nq, G, H, D = q.shape
    kt = np.ascontiguousarray(k_tok, dtype=np.uint16)
    vt = np.ascontiguousarray(v_tok, dtype=np.uint16)
    assert kt.shape == vt.shape and kt.shape[1:] == (G, D) and kt.shape[0] >= n_kv
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    assert ids.shape[:2] == (G, nq)
    k = ids.shape[2]
    out = np.empty((nq, G, H, D))
    B = np.empty((nq, G, H, D))
    rc = lib().oracle_attention(_p(q), G * H * D, _p(kt), _p(vt), G * D, _p(ids), k, G, nq, H, D,
                                n_kv, bs, k, _p(out), _p(B))
    assert rc == 0
    return out, B


def check_attention(o_dev: np.ndarray, ref: np.ndarray, B: np.ndarray) -> CheckResult:
    """Every output element within its bound (elements with B = 0 exactly)."""
    return check_scores(np.asarray(o_dev, dtype=np.float64).reshape(-1, ref.shape[-1]),
                        Scores(ref.reshape(-1, ref.shape[-1]), np.zeros(1), B.reshape(-1, ref.shape[-1]),
                               np.zeros(1, np.int64)))


# --------------------------------------------------------------------------
# Checker (R4-R7)
# --------------------------------------------------------------------------

@dataclass
class CheckResult:
    ok: bool
    utilisation: float   # max |err| / B over cells with B > 0
    n_fail: int
    n_cells: int
    worst: tuple | None  # (row index, block, s_gpu, score_ref, B)

    def __str__(self):
        return (f"ok={self.ok} util={100 * self.utilisation:.3f}% fail={self.n_fail}/"
                f"{self.n_cells} worst={self.worst}")


def check_scores(s_gpu: np.ndarray, ref: Scores) -> CheckResult:
    """R4: every cell within B; cells with B == 0 must be exactly equal."""
    s = np.asarray(s_gpu, dtype=np.float64)
    assert s.shape == ref.score.shape, (s.shape, ref.score.shape)
    err = np.abs(s - ref.score)
    bad = ~(err <= ref.B)          # NaN counts as a failure
    with np.errstate(divide="ignore", invalid="ignore"):
        util = np.where(ref.B > 0, err / ref.B, np.where(err == 0, 0.0, np.inf))
    n_fail = int(bad.sum())
    worst = None
    umax = 0.0
    if s.size:
        idx = np.unravel_index(int(np.nanargmax(np.where(np.isnan(util), np.inf, util))), s.shape)
        umax = float(util[idx])
        worst = (int(idx[0]), int(idx[1]), float(s[idx]), float(ref.score[idx]), float(ref.B[idx]))
    return CheckResult(n_fail == 0, umax, n_fail, int(s.size), worst)


def negative_controls(ref: Scores, s_gpu: np.ndarray, seed: int = 7) -> tuple[bool, bool]:
    """R5: (i) +2.5*B on every cell with B > 0, (ii) +2.5*B on one seeded cell
    with B > 0.  Returns (i_failed, ii_failed): both must be True."""
    s = np.asarray(s_gpu, dtype=np.float64)
    pos = ref.B > 0
    if not pos.any():
        return True, True
    p1 = s + NEG_CONTROL * ref.B * pos
    f1 = not check_scores(p1, ref).ok
    cand = np.flatnonzero(pos.ravel())
    rng = np.random.default_rng(seed)
    c = int(cand[rng.integers(cand.size)])
    p2 = s.copy().ravel()
    p2[c] = ref.score.ravel()[c] + NEG_CONTROL * ref.B.ravel()[c]
    f2 = not check_scores(p2.reshape(s.shape), ref).ok
    return f1, f2


@dataclass
class SelectionResult:
    ok: bool
    rows_differing: int
    ids_differing: int
    n_ids: int
    worst_gap_ratio: float  # max over swapped pairs of gap / (2*max(B))
    detail: str = ""


def near_tie_limit(b_x: float, b_y: float) -> float:
    """Largest score_ref gap by which a device selection may prefer block x
    over block y: NEAR_TIE_FACTOR times the larger of the two bounds (either
    cell's score may be off by its own B, so the guard must admit the wider
    one)."""
    return NEAR_TIE_FACTOR * max(b_x, b_y)


def check_selection(ids_gpu: np.ndarray, ref: Scores, k: int) -> SelectionResult:
    """R6: the device ids against the oracle's own top-k of score_ref.  Per row
    the sets must match, except that every x in gpu\\oracle and y in
    oracle\\gpu satisfy score_ref(y) - score_ref(x) <= 2*max(B(x), B(y)).
    Slots past min(k, nb) must be -1 in both."""
    ids_gpu = np.asarray(ids_gpu, dtype=np.int64)
    ids_ref, _ = topk(ref.score, k)
    nb = ref.score.shape[1]
    kk = min(k, nb)
    rows_diff = ids_diff = 0
    worst = 0.0
    ok = True
    detail = ""
    for r in range(ids_gpu.shape[0]):
        g = ids_gpu[r]
        o = ids_ref[r].astype(np.int64)
        if np.any(g[kk:] != -1):
            ok = False
            detail = f"row {r}: padding not -1"
            continue
        gs, os_ = set(g[:kk].tolist()), set(o[:kk].tolist())
        if len(gs) != kk or any(x < 0 or x >= nb for x in gs):
            ok = False
            detail = f"row {r}: invalid or duplicate ids {g[:kk]}"
            continue
        xs, ys = gs - os_, os_ - gs
        if xs:
            rows_diff += 1
            ids_diff += len(xs)
            for x in xs:
                for y in ys:
                    gap = ref.score[r, y] - ref.score[r, x]
                    lim = near_tie_limit(float(ref.B[r, x]), float(ref.B[r, y]))
                    if gap > lim:
                        ok = False
                        detail = f"row {r}: swapped {x}<->{y} gap {gap} > {lim}"
                    if lim > 0:
                        worst = max(worst, gap / lim)
                    elif gap > 0:
                        worst = np.inf
    return SelectionResult(ok, rows_diff, ids_diff, ids_gpu.shape[0] * kk, worst, detail)

