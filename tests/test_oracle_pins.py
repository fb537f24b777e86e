"""CPU pins of the float64 oracle.

Each test ties the oracle to something other than itself: exact rational
arithmetic on tiny inputs, numpy's float64 matmul in the single-head case,
closed forms of coded fixtures, hand-worked golden examples, invariants of the
formula, the x86 F16C conversion instruction, numpy's sequential float32
accumulation, and an O(n^2) rank count for the top-k order.

The formula is the QSA block score of Strata pull request #228 (part 1, first
paragraph): score(t, b) = sum_h relu(sum_i k_b[i] * q_{t,h}[i]); the bound is
the same page's arithmetic contract.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
import qsa_inputs as qi

HERE = os.path.dirname(os.path.abspath(__file__))


# --------------------------------------------------------------------------
# helpers independent of the oracle
# --------------------------------------------------------------------------

def f16_bits_to_int24(b: int) -> int:
    """fp16 bits -> integer m with value m * 2^-24 (finite values only),
    from the bit fields of IEEE 754 binary16."""
    s, e, m = (b >> 15) & 1, (b >> 10) & 0x1F, b & 0x3FF
    assert e != 31
    v = m if e == 0 else (1024 + m) << (e - 1)
    return -v if s else v


def exact_scores(q16: np.ndarray, kblk: np.ndarray, nb: int):
    """Exact score and S as Fractions, by integer arithmetic."""
    nq, G, H, D = q16.shape
    qi_ = np.vectorize(f16_bits_to_int24, otypes=[object])(q16.astype(np.int64))
    ki_ = np.vectorize(f16_bits_to_int24, otypes=[object])(kblk.astype(np.int64))
    scale = Fraction(1, 2 ** 48)
    sc = np.empty((G * nq, nb), dtype=object)
    S = np.empty((G * nq, nb), dtype=object)
    for g in range(G):
        for t in range(nq):
            for b in range(nb):
                tot = 0
                sabs = 0
                for h in range(H):
                    d = 0
                    for i in range(D):
                        p = int(ki_[g, b, i]) * int(qi_[t, g, h, i])
                        d += p
                        sabs += abs(p)
                    tot += max(d, 0)
                sc[g * nq + t, b] = tot * scale
                S[g * nq + t, b] = sabs * scale
    return sc, S


SPECIAL_F16 = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x83FF, 0x0400, 0x8400,
                        0x7BFF, 0xFBFF, 0x3C00, 0xBC00, 0x3555, 0x0200], dtype=np.uint16)


def random_f16(rng, shape, special_frac=0.2):
    """fp16 bits: mostly random finite values of mixed magnitude, some special."""
    n = int(np.prod(shape))
    e = rng.integers(0, 31, n)            # every finite exponent incl. subnormal
    m = rng.integers(0, 1024, n)
    s = rng.integers(0, 2, n)
    bits = ((s << 15) | (e << 10) | m).astype(np.uint16)
    pick = rng.random(n) < special_frac
    bits[pick] = SPECIAL_F16[rng.integers(0, SPECIAL_F16.size, int(pick.sum()))]
    return bits.reshape(shape)


# --------------------------------------------------------------------------
# fp16 decoding and conversion
# --------------------------------------------------------------------------

def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.f16_to_f64(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))  # -0 kept


def test_int24_helper_matches_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    fin = np.isfinite(bits.view(np.float16))
    vals = [f16_bits_to_int24(int(b)) * 2.0 ** -24 for b in bits[fin]]
    assert np.array_equal(np.array(vals), bits[fin].view(np.float16).astype(np.float64))


@pytest.fixture(scope="module")
def f16c_lib(tmp_path_factory):
    src = os.path.join(HERE, "pins", "f16c_ref.c")
    out = str(tmp_path_factory.mktemp("f16c") / "libf16c.so")
    subprocess.run(["gcc", "-O2", "-mf16c", "-fopenmp", "-fPIC", "-shared", "-o", out, src],
                   check=True)
    L = ctypes.CDLL(out)
    L.f16c_compare_range.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.POINTER(ctypes.c_uint64)]
    L.f16c_compare_range.restype = ctypes.c_int64
    L.f16c_one.argtypes = [ctypes.c_float]
    L.f16c_one.restype = ctypes.c_uint16
    return L


def test_convert_exhaustive_vs_f16c(f16c_lib):
    """The oracle's hand-written fp32 -> fp16 (nearest even) equals the F16C
    instruction on all 2^32 fp32 bit patterns, NaNs included."""
    fn = ctypes.cast(oracle.lib().oracle_f32_to_f16_one, ctypes.c_void_p)
    first = ctypes.c_uint64()
    bad = f16c_lib.f16c_compare_range(fn, 0, 1 << 32, ctypes.byref(first))
    assert bad == 0, f"{bad} mismatches, first pattern {first.value:#010x}"


def test_convert_vs_numpy_nonnan():
    """Same converter against numpy's float32 -> float16 on non-NaN samples."""
    rng = np.random.default_rng(5)
    pats = np.concatenate([
        rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64),
        # every exponent with the fraction patterns around the rounding points
        (np.arange(512, dtype=np.uint64)[:, None] << np.uint64(23)
         | np.array([0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001, 0x3000,
                     0x7FFFFF, 0x7FE000, 0x7FF000], dtype=np.uint64)[None, :]).ravel(),
    ]).astype(np.uint32)
    x = pats.view(np.float32)
    x = x[~np.isnan(x)]
    got = oracle.convert_f32_f16(x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_convert_known_values():
    cases = {1.0: 0x3C00, -2.0: 0xC000, 65504.0: 0x7BFF, 65519.996: 0x7BFF, 65520.0: 0x7C00,
             2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000, 2.0 ** -25 * 1.0000001: 0x0001,
             3 * 2.0 ** -25: 0x0002, 2.0 ** -14: 0x0400, 1.0 + 2.0 ** -11: 0x3C00,
             1.0 + 3 * 2.0 ** -11: 0x3C02, -0.0: 0x8000, float("inf"): 0x7C00}
    for v, bits in cases.items():
        assert oracle.lib().oracle_f32_to_f16_one(v) == bits, (v, hex(bits))


# --------------------------------------------------------------------------
# scores: exact brute force, library special case, closed forms, invariants
# --------------------------------------------------------------------------

# Each pin below is a function of the scoring routine it checks, so that the
# same pins can be run against deliberately broken scorers (planted mistakes
# in test_planted_mistakes.py), which each must fail at least one of them.

def pin_exact_bruteforce(scores_fn, seed: int) -> None:
    rng = np.random.default_rng(100 + seed)
    D = [1, 2, 3, 16, 64][seed % 5]
    G, nq, H, nb = int(rng.integers(1, 3)), int(rng.integers(1, 6)), int(rng.integers(1, 5)), \
        int(rng.integers(1, 6))
    if seed % 4 == 3:   # several KV heads and query heads: layout mistakes show
        G, H = 2, max(H, 2)
    q16 = random_f16(rng, (nq, G, H, D))
    kb = random_f16(rng, (G, nb, D))
    ref = scores_fn(q16, kb, nb)
    ex, exS = exact_scores(q16, kb, nb)
    for r in range(G * nq):
        for b in range(nb):
            s_ex, S_ex = ex[r, b], exS[r, b]
            tol = float(S_ex) * 2.0 ** -45
            assert abs(Fraction(ref.score[r, b]) - s_ex) <= Fraction(tol), (r, b)
            assert abs(Fraction(ref.S[r, b]) - S_ex) <= Fraction(tol), (r, b)
            want_B = oracle.BOUND_REL * float(S_ex) + oracle.BOUND_ABS * float(s_ex)
            assert math.isclose(ref.B[r, b], want_B, rel_tol=1e-12, abs_tol=1e-300)


@pytest.mark.parametrize("seed", range(12))
def test_scores_vs_exact_bruteforce(seed):
    pin_exact_bruteforce(oracle.scores, seed)


def pin_single_head_matmul(scores_fn) -> None:
    """With H = 1 the score is relu(Q K^T): numpy float64 matmul."""
    rng = np.random.default_rng(3)
    nq, nb, D = 33, 47, 128
    q16 = qi.f64_to_f16_bits(rng.standard_normal((nq, 1, 1, D)) / math.sqrt(D))
    kb = qi.f64_to_f16_bits(rng.standard_normal((1, nb, D)) / math.sqrt(D))
    ref = scores_fn(q16, kb, nb)
    Q = q16.view(np.float16).astype(np.float64).reshape(nq, D)
    K = kb.view(np.float16).astype(np.float64).reshape(nb, D)
    want = np.maximum(Q @ K.T, 0.0)
    assert np.all(np.abs(ref.score - want) <= D * 2.0 ** -52 * ref.S)
    # S of one head is the matmul of the magnitudes
    assert np.all(np.abs(ref.S - np.abs(Q) @ np.abs(K).T) <= D * 2.0 ** -52 * ref.S)


def test_single_head_is_relu_matmul():
    pin_single_head_matmul(oracle.scores)


def pin_coded_fixture(scores_fn) -> None:
    cfg = qi.CONFIGS["nq256_nkv32768"]
    small = qi.Config("coded_small", 2, 40, cfg.H, cfg.D, 64 * 37, 64, 8, "normal", 0)
    w = qi.coded_fixture(small)
    ref = scores_fn(w.q16, w.kblk, small.nb)
    ch, kint = w.extra["channel"], w.extra["kint"]
    want = np.zeros((small.G * small.nq, small.nb))
    for g in range(small.G):
        for t in range(small.nq):
            want[g * small.nq + t] = np.maximum(kint[g, :small.nb, ch[t]], 0).sum(axis=0)
    assert np.array_equal(ref.score, want)
    assert np.array_equal(ref.S, np.abs(kint[:, :small.nb, :][
        np.repeat(np.arange(small.G), small.nq)[:, None, None],
        np.arange(small.nb)[None, :, None], np.tile(ch, (small.G, 1))[:, None, :]]).sum(axis=2))


def test_coded_fixture_closed_form():
    pin_coded_fixture(oracle.scores)


def pin_integer_fixture(scores_fn) -> None:
    cfg = qi.Config("int_small", 2, 19, 8, 128, 64 * 9 + 7, 64, 8, "normal", 0)
    w = qi.integer_fixture(cfg)
    ref = scores_fn(w.q16, w.kblk, cfg.nb)
    Q = w.q16.view(np.float16).astype(np.int64)
    K = w.kblk.view(np.float16).astype(np.int64)
    want = np.zeros((cfg.G * cfg.nq, cfg.nb), dtype=np.int64)
    for g in range(cfg.G):
        d = np.einsum("thi,bi->thb", Q[:, g], K[g, :cfg.nb])
        want[g * cfg.nq:(g + 1) * cfg.nq] = np.maximum(d, 0).sum(axis=1)
    assert np.array_equal(ref.score, want.astype(np.float64))
    assert want.max() > 2048  # large enough that fp16 accumulation would fail
    wantS = np.zeros_like(want)
    for g in range(cfg.G):
        wantS[g * cfg.nq:(g + 1) * cfg.nq] = np.einsum("thi,bi->tb", np.abs(Q[:, g]),
                                                       np.abs(K[g, :cfg.nb]))
    assert np.array_equal(ref.S, wantS.astype(np.float64))
    assert np.allclose(ref.B, oracle.BOUND_REL * ref.S + oracle.BOUND_ABS * ref.score,
                       rtol=1e-14, atol=0)


def test_integer_fixture_exact():
    pin_integer_fixture(oracle.scores)


def pin_trivial_closed_forms(scores_fn) -> None:
    rng = np.random.default_rng(9)
    nq, G, H, D, nb = 5, 2, 3, 64, 11
    kb = qi.f64_to_f16_bits(rng.standard_normal((G, nb, D)))
    zero_q = np.zeros((nq, G, H, D), np.uint16)
    ref = scores_fn(zero_q, kb, nb)
    assert np.all(ref.score == 0) and np.all(ref.S == 0) and np.all(ref.B == 0)
    ids, _ = oracle.topk(ref.score, 4)
    assert np.array_equal(ids, np.tile(np.arange(4, dtype=np.int32), (G * nq, 1)))
    # all key rows equal -> equal scores -> ids 0..k-1
    q16 = qi.f64_to_f16_bits(rng.standard_normal((nq, G, H, D)))
    same = np.repeat(kb[:, :1, :], nb, axis=1)
    ref = scores_fn(q16, same, nb)
    assert np.all(ref.score == ref.score[:, :1])
    ids, _ = oracle.topk(ref.score, 4)
    assert np.array_equal(ids, np.tile(np.arange(4, dtype=np.int32), (G * nq, 1)))
    # one dominant block: q = |k_b*| direction on every head
    kd = kb.copy()
    kd[:, 7, :] = qi.f64_to_f16_bits(np.full((G, D), 4.0))
    qp = qi.f64_to_f16_bits(np.abs(rng.standard_normal((nq, G, H, D))) + 1.0)
    kd[:, :7] = qi.f64_to_f16_bits(np.full((G, 7, D), -1.0))
    kd[:, 8:] = qi.f64_to_f16_bits(np.full((G, nb - 8, D), -1.0))
    ref = scores_fn(qp, kd, nb)
    ids, _ = oracle.topk(ref.score, 1)
    assert np.all(ids[:, 0] == 7)


def test_trivial_closed_forms():
    pin_trivial_closed_forms(oracle.scores)


def pin_invariants(scores_fn) -> None:
    rng = np.random.default_rng(11)
    nq, G, H, D, nb = 7, 2, 4, 64, 13
    q16 = qi.f64_to_f16_bits(rng.standard_normal((nq, G, H, D)) * 0.3)
    kb = qi.f64_to_f16_bits(rng.standard_normal((G, nb, D)) * 0.3)
    ref = scores_fn(q16, kb, nb)
    assert np.all(ref.score >= 0) and np.all(ref.score <= ref.S)
    # head permutation: same value up to float64 summation order
    perm = rng.permutation(H)
    rp = scores_fn(q16[:, :, perm], kb, nb)
    assert np.all(np.abs(rp.score - ref.score) <= 2.0 ** -45 * ref.S)
    # block permutation: each block is independent
    bp = rng.permutation(nb)
    rb = scores_fn(q16, kb[:, bp], nb)
    assert np.array_equal(rb.score, ref.score[:, bp])
    # scaling by 2^j scales scores by 2^(2j) exactly
    q2 = qi.f64_to_f16_bits(q16.view(np.float16).astype(np.float64) * 4.0)
    k2 = qi.f64_to_f16_bits(kb.view(np.float16).astype(np.float64) * 0.5)
    r2 = scores_fn(q2, k2, nb)
    assert np.array_equal(r2.score, ref.score * 2.0)
    # relu(x) - relu(-x) = x: score(Q,K) - score(Q,-K) = (sum_h q_h) . k
    kneg = kb ^ np.uint16(0x8000)
    rn = scores_fn(q16, kneg, nb)
    Qf = q16.view(np.float16).astype(np.float64)
    Kf = kb.view(np.float16).astype(np.float64)
    for g in range(G):
        want = Qf[:, g].sum(axis=1) @ Kf[g].T
        got = ref.score[g * nq:(g + 1) * nq] - rn.score[g * nq:(g + 1) * nq]
        assert np.all(np.abs(got - want) <= 2.0 ** -44 * ref.S[g * nq:(g + 1) * nq])


def test_invariants():
    pin_invariants(oracle.scores)


def pin_f32_queries(scores_fn) -> None:
    """For fp32 queries the oracle uses the fp32 values themselves."""
    rng = np.random.default_rng(4)
    nq, G, H, D, nb = 3, 1, 2, 64, 5
    q32 = (rng.standard_normal((nq, G, H, D)) / 8).astype(np.float32)
    kb = qi.f64_to_f16_bits(rng.standard_normal((G, nb, D)) / 8)
    ref = scores_fn(q32, kb, nb)
    Q = q32.astype(np.float64)
    K = kb.view(np.float16).astype(np.float64)
    want = np.maximum(np.einsum("thi,bi->thb", Q[:, 0], K[0]), 0).sum(axis=1)
    assert np.all(np.abs(ref.score - want) <= 2.0 ** -45 * ref.S)


def test_f32_queries_use_unrounded_values():
    pin_f32_queries(oracle.scores)


# --------------------------------------------------------------------------
# golden hand-worked examples
# --------------------------------------------------------------------------

def load_hand_examples():
    path = os.path.join(HERE, "golden", "hand_examples.txt")
    exs, cur = [], None
    for line in open(path):
        line = line.split("#", 1)[0].split()
        if not line:
            continue
        tag = line[0]
        if tag == "example":
            kv = dict(zip(line[2::2], map(int, line[3::2])))
            cur = dict(name=line[1], **kv, q={}, kb={}, score={}, S={}, topk={})
        elif tag == "q":
            cur["q"][(int(line[1]), int(line[2]))] = [float(x) for x in line[3:]]
        elif tag in ("kb", "score", "S", "topk"):
            cur[tag][int(line[1])] = [float(x) for x in line[2:]]
        elif tag == "end":
            exs.append(cur)
    return exs


def pin_hand_example(scores_fn, ex) -> None:
    H, D, nq, nb, k = ex["H"], ex["D"], ex["nq"], ex["nb"], ex["k"]
    q = np.zeros((nq, 1, H, D))
    for (t, h), v in ex["q"].items():
        q[t, 0, h] = v
    kb = np.array([ex["kb"][b] for b in range(nb)])[None]
    ref = scores_fn(qi.f64_to_f16_bits(q), qi.f64_to_f16_bits(kb), nb)
    for t in range(nq):
        assert ref.score[t].tolist() == ex["score"][t]
        assert ref.S[t].tolist() == ex["S"][t]
    ids, _ = oracle.topk(ref.score, k)
    for t in range(nq):
        assert ids[t].tolist() == [int(x) for x in ex["topk"][t]]


@pytest.mark.parametrize("ex", load_hand_examples(), ids=lambda e: e["name"])
def test_hand_examples(ex):
    pin_hand_example(oracle.scores, ex)


def test_contract_constants_match_pages():
    vals = {}
    for line in open(os.path.join(HERE, "golden", "contract.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            key, v = [x.strip() for x in line.split("=")]
            vals[key] = float(v)
    assert oracle.BOUND_REL == 2.0 ** vals["bound_rel_log2"]
    assert oracle.BOUND_ABS == vals["bound_abs_coeff"] * 2.0 ** vals["bound_abs_log2"]
    assert oracle.NEG_CONTROL == vals["negative_control_factor"]
    assert oracle.NEAR_TIE_FACTOR == vals["near_tie_factor"]
    assert oracle.near_tie_limit(1.0, 0.5) == vals["near_tie_factor"]


# --------------------------------------------------------------------------
# fixed-order fp32 block model (the tail kernel's contract)
# --------------------------------------------------------------------------

def test_block_model_vs_numpy_sequential_float32():
    """numpy's add.accumulate is a strictly sequential float32 sum; products of
    two fp16 values are exact in float32, so fmaf(k, q, acc) and
    round(acc + k*q) coincide and the model must equal it bit for bit."""
    rng = np.random.default_rng(21)
    nq, G, H, D, nb = 9, 2, 8, 128, 4
    q16 = qi.f64_to_f16_bits(rng.standard_normal((nq, G, H, D)) / math.sqrt(D))
    kb = qi.f64_to_f16_bits(rng.standard_normal((G, nb, D)) / math.sqrt(D))
    b = 3
    got = oracle.block_model_f32(q16, kb, b)
    Q = q16.view(np.float16).astype(np.float32)
    K = kb.view(np.float16).astype(np.float32)
    want = np.empty(G * nq, np.float32)
    for g in range(G):
        for t in range(nq):
            prods = K[g, b][None, :] * Q[t, g]                  # exact, [H][D]
            acc = np.add.accumulate(prods, axis=1, dtype=np.float32)[:, -1]
            r = np.where(acc > 0, acc, np.float32(0))
            want[g * nq + t] = np.add.accumulate(np.concatenate([[np.float32(0)], r]),
                                                 dtype=np.float32)[-1]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_block_model_integer_exact_and_within_bound():
    cfg = qi.Config("int_tail", 1, 11, 8, 128, 64 * 3 + 5, 64, 4, "normal", 0)
    w = qi.integer_fixture(cfg)
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    got = oracle.block_model_f32(w.q16, w.kblk, cfg.nb - 1)
    assert np.array_equal(got.astype(np.float64), ref.score[:, -1])
    wr = qi.make(qi.TINY)
    refr = oracle.scores(wr.q16, wr.kblk, wr.cfg.nb)
    gr = oracle.block_model_f32(wr.q16, wr.kblk, wr.cfg.nb - 1)
    assert np.all(np.abs(gr - refr.score[:, -1]) <= refr.B[:, -1])


def test_block_model_x8_is_exactly_64x():
    w = qi.make(qi.TINY)
    w8 = qi.scaled_by_8(w)
    b = w.cfg.nb - 1
    a = oracle.block_model_f32(w.q16, w.kblk, b)
    a8 = oracle.block_model_f32(w8.q16, w8.kblk, b)
    assert np.array_equal(a8, a * np.float32(64))


# --------------------------------------------------------------------------
# top-k order
# --------------------------------------------------------------------------

def rank_count_topk(row: np.ndarray, k: int) -> list[int]:
    """O(n^2): rank(b) = #{b' better than b}; NaN below every number."""
    n = row.size

    def better(a, b):  # is a better than b
        sa, sb = row[a], row[b]
        na, nb_ = math.isnan(sa), math.isnan(sb)
        if na != nb_:
            return nb_
        if not na and sa != sb:
            return sa > sb
        return a < b

    ranks = [sum(better(o, b) for o in range(n)) for b in range(n)]
    order = sorted(range(n), key=lambda b: ranks[b])
    return [order[j] if j < n else -1 for j in range(k)]


@pytest.mark.parametrize("seed", range(6))
def test_topk_vs_rank_count(seed):
    rng = np.random.default_rng(300 + seed)
    rows, nb = 6, int(rng.integers(1, 90))
    s = rng.integers(-3, 4, (rows, nb)).astype(np.float64) * 0.5
    s[rng.random((rows, nb)) < 0.1] = -0.0
    s[rng.random((rows, nb)) < 0.05] = np.nan
    s[rng.random((rows, nb)) < 0.05] = np.inf
    for k in (0, 1, 5, 64, nb + 3):
        ids, vals = oracle.topk(s, k)
        for r in range(rows):
            assert ids[r].tolist() == rank_count_topk(s[r], k)
            sel = ids[r] >= 0
            assert np.array_equal(vals[r][sel], s[r][ids[r][sel]], equal_nan=True)
            assert np.all(vals[r][~sel] == -np.inf)


def test_topk_empty_row():
    ids, vals = oracle.topk(np.zeros((3, 0)), 4)
    assert np.all(ids == -1) and np.all(vals == -np.inf)


# --------------------------------------------------------------------------
# checker
# --------------------------------------------------------------------------

def test_checker_bound_edges_and_negative_controls():
    w = qi.make(qi.TINY)
    ref = oracle.scores(w.q16, w.kblk, w.cfg.nb)
    s = ref.score.astype(np.float32).astype(np.float64)
    assert oracle.check_scores(s, ref).ok
    sign = np.where(np.random.default_rng(1).random(s.shape) < 0.5, -1.0, 1.0)
    assert oracle.check_scores(ref.score + 0.99 * ref.B * sign, ref).ok
    r = oracle.check_scores(ref.score + 1.01 * ref.B * sign, ref)
    assert not r.ok and r.n_fail == s.size
    f1, f2 = oracle.negative_controls(ref, s)
    assert f1 and f2
    # exact-mode cells (B == 0) tolerate nothing
    z = oracle.Scores(np.zeros((1, 2)), np.zeros((1, 2)), np.zeros((1, 2)), np.zeros(1, np.int64))
    assert oracle.check_scores(np.zeros((1, 2)), z).ok
    assert not oracle.check_scores(np.array([[0.0, 1e-30]]), z).ok
    assert not oracle.check_scores(np.array([[0.0, np.nan]]), z).ok


def test_selection_checker_near_ties():
    w = qi.make(qi.TINY)
    ref = oracle.scores(w.q16, w.kblk, w.cfg.nb)
    ids, _ = oracle.topk(ref.score, 4)
    assert oracle.check_selection(ids, ref, 4).ok
    bad = ids.copy()
    bad[0, 0] = bad[0, 1]  # duplicate id
    assert not oracle.check_selection(bad, ref, 4).ok
    bad = ids.copy()
    bad[1, 2] = w.cfg.nb   # id out of range
    assert not oracle.check_selection(bad, ref, 4).ok


def _one_row(score, B, ids, k):
    """A single-row oracle.Scores with given score_ref and B, and the device
    ids to judge."""
    score = np.array([score], dtype=np.float64)
    B = np.array([B], dtype=np.float64)
    return (np.array([ids], dtype=np.int64), oracle.Scores(score, np.zeros_like(score), B,
                                                           np.zeros(1, np.int64)), k)


# Gaps just inside and just outside 2*max(B), exact binary fractions.
_IN, _OUT = 127.0 / 64.0, 129.0 / 64.0   # 1.984..., 2.016... times max(B)


def selection_pins():
    """(name, ids, Scores, k, verdict) rows worked by hand from the near-tie
    rule: the oracle's top-2 of score_ref is {0, 1}; the device picked
    block 2 instead of block 1 (or agrees).  The swap is allowed iff
    score_ref(1) - score_ref(2) <= 2 * max(B(1), B(2))."""
    s = 10.0
    return [
        ("agree", *_one_row([20.0, s, s - 5.0, 0.0], [1, 1, 1, 1], [0, 1], 2), True),
        ("agree_order_free", *_one_row([20.0, s, s - 5.0, 0.0], [1, 1, 1, 1], [1, 0], 2), True),
        # equal bounds: just inside passes, just outside fails
        ("inside_equal_B", *_one_row([20.0, s, s - _IN, 0.0], [1, 1, 1, 1], [0, 2], 2), True),
        ("outside_equal_B", *_one_row([20.0, s, s - _OUT, 0.0], [1, 1, 1, 1], [0, 2], 2), False),
        # unequal bounds: the larger one decides, whichever cell holds it
        ("inside_max_at_x", *_one_row([20.0, s, s - _IN, 0.0], [1, 0.125, 1, 1], [0, 2], 2), True),
        ("inside_max_at_y", *_one_row([20.0, s, s - _IN, 0.0], [1, 1, 0.125, 1], [0, 2], 2), True),
        ("outside_max_at_x", *_one_row([20.0, s, s - _OUT, 0.0], [1, 0.125, 1, 1], [0, 2], 2),
         False),
        ("outside_max_at_y", *_one_row([20.0, s, s - _OUT, 0.0], [1, 1, 0.125, 1], [0, 2], 2),
         False),
        # the sum of the two bounds is wider than the rule: 2.016 < 2.25
        ("outside_not_sum", *_one_row([20.0, s, s - _OUT, 0.0], [1, 1, 0.125, 1], [0, 2], 2),
         False),
        # exact cells (B == 0): an exact tie may go either way, any gap may not
        ("exact_tie_either_way", *_one_row([20.0, s, s, 0.0], [0, 0, 0, 0], [0, 2], 2), True),
        ("exact_gap_fails", *_one_row([20.0, s, s - 2.0 ** -40, 0.0], [0, 0, 0, 0], [0, 2], 2),
         False),
        # k > nb pads with -1; a real id in a pad slot fails
        ("pads", *_one_row([1.0, 2.0], [0, 0], [1, 0, -1], 3), True),
        ("pad_not_minus1", *_one_row([1.0, 2.0], [0, 0], [1, 0, 0], 3), False),
        # two swaps in one row: each pair (x, y) is judged
        ("two_swaps_inside", *_one_row([20.0, s, s, s - _IN, s - _IN], [1, 1, 1, 1, 1],
                                       [0, 3, 4], 3), True),
        ("two_swaps_one_outside", *_one_row([20.0, s, s, s - _IN, s - _OUT], [1, 1, 1, 1, 1],
                                            [0, 3, 4], 3), False),
    ]


@pytest.mark.parametrize("pin", selection_pins(), ids=lambda p: p[0])
def test_selection_checker_hand_rows(pin):
    name, ids, ref, k, verdict = pin
    res = oracle.check_selection(ids, ref, k)
    assert res.ok == verdict, (name, res.detail)


def selection_pins_hold() -> bool:
    return all(oracle.check_selection(ids, ref, k).ok == verdict
               for _, ids, ref, k, verdict in selection_pins())


@pytest.mark.parametrize("mutant", [
    ("factor_4", lambda bx, by: 4.0 * max(bx, by)),
    ("factor_1", lambda bx, by: 1.0 * max(bx, by)),
    ("min_of_bounds", lambda bx, by: 2.0 * min(bx, by)),
    ("bound_of_x_only", lambda bx, by: 2.0 * bx),
    ("bound_of_y_only", lambda bx, by: 2.0 * by),
    ("sum_of_bounds", lambda bx, by: 2.0 * (bx + by)),
    ("reject_every_swap", lambda bx, by: -1.0),
    ("accept_every_swap", lambda bx, by: np.inf),
], ids=lambda m: m[0])
def test_selection_pins_catch_planted_checker_mistakes(mutant, monkeypatch):
    """Each plausible mistake in the near-tie rule, planted into the checker,
    makes at least one hand row come out wrong."""
    assert selection_pins_hold()
    monkeypatch.setattr(oracle, "near_tie_limit", mutant[1])
    assert not selection_pins_hold(), mutant[0]


# --------------------------------------------------------------------------
# input generators (shared module, holds no arithmetic of the method)
# --------------------------------------------------------------------------

def test_splitmix64_published_values():
    """First outputs of splitmix64 from state 1234567 (the widely published
    reference sequence of Vigna's splitmix64.c)."""
    got = qi.splitmix64(1234567, 0, 0, 5).tolist()
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_stream_slices_are_consistent():
    a = qi.splitmix64(77, 3, 0, 1000)
    b = qi.splitmix64(77, 3, 400, 300)
    assert np.array_equal(a[400:700], b)
    n = qi.normal(5, 1, 10001)
    assert abs(n.mean()) < 0.05 and abs(n.std() - 1) < 0.05


def test_config_shapes():
    c = qi.CONFIGS
    assert (qi.TINY.nb, qi.TINY.nf) == (16, 15)
    assert c["nq256_nkv4096"].nb == 64 and c["nq256_nkv32768"].nb == 512
    assert c["nq256_nkv131072"].nb == 2048
    assert (qi.PREFILL.nb, qi.PREFILL.nf, qi.PREFILL.rows) == (2049, 2048, 65536)
    assert qi.PREFILL.flop == 2 * 65536 * 8 * 128 * 2049
    w = qi.make(qi.TINY)
    assert w.q16.shape == (37, 1, 4, 64) and w.kblk.shape == (1, 16, 64)
    x8 = qi.scaled_by_8(qi.make("nq256_nkv4096"))
    assert np.abs(x8.q16.view(np.float16).astype(np.float64)).max() < 8188


# --------------------------------------------------------------------------
# block keys: the mean of a block's token keys, rounded once to fp16 (the
# reading taken for k_b, which the pages index but never define)
# --------------------------------------------------------------------------

def f16_nearest_fraction(x: Fraction) -> int:
    """fp16 bits of the value of the fp16 grid nearest to x, ties to the even
    significand, from the format's definition (finite x, |x| < 65520):
    binade [2^E, 2^(E+1)) has spacing 2^(E-10) for E >= -14, and below 2^-14
    the spacing is 2^-24."""
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return 0
    E = 15
    while E > -14 and a < Fraction(2) ** E:
        E -= 1
    spacing = Fraction(2) ** (E - 10)
    q, r = divmod(a, spacing)
    q = int(q)
    if r * 2 > spacing or (r * 2 == spacing and q % 2 == 1):
        q += 1
    if q < 1024:                      # subnormal (E = -14, below 2^-14)
        return sign | q
    if q == 2048:
        q, E = 1024, E + 1
    if E > 15:
        return sign | 0x7C00
    return sign | ((E + 15) << 10) | (q - 1024)


def test_round_ratio_vs_fractions():
    rng = np.random.default_rng(77)
    cases = [(1, 2), (3, 2), (5, 2), (-1, 2), (1 << 24, 3), (-(1 << 24), 3), (2047, 1),
             (2049, 2), (2 ** 40 - 1, 1), (65504 << 24, 1), (1023 * 2 + 1, 2), (1 << 10, 1),
             ((1 << 10) * 3 - 1, 3)]
    for _ in range(3000):
        den = int(rng.integers(1, 9000))
        num = int(rng.integers(-(2 ** 40), 2 ** 40)) * int(rng.integers(1, den + 1)) // den
        if rng.random() < 0.3:
            num = int(rng.integers(-3000, 3000))          # subnormal range and ties
        cases.append((num, den))
    for num, den in cases:
        want = f16_nearest_fraction(Fraction(num, den) / 2 ** 24)
        assert oracle.round_ratio_f16(num, den) == want, (num, den, hex(want))


def _keys_fraction(k_tok, n_kv, bs):
    n, G, D = k_tok.shape
    nb = -(-n_kv // bs)
    vals = k_tok.view(np.float16).astype(np.float64)
    out = np.zeros((G, nb, D), np.uint16)
    for g in range(G):
        for b in range(nb):
            t0, t1 = b * bs, min((b + 1) * bs, n_kv)
            for i in range(D):
                s = sum((Fraction(float(v)) for v in vals[t0:t1, g, i]), Fraction(0))
                out[g, b, i] = f16_nearest_fraction(s / (t1 - t0))
    return out


@pytest.mark.parametrize("n_kv,bs,G,D", [(13, 3, 2, 5), (40, 7, 1, 8), (64 * 3 + 5, 64, 2, 4),
                                         (1, 64, 1, 3), (0, 64, 2, 4)])
def test_block_keys_vs_fractions(n_kv, bs, G, D):
    rng = np.random.default_rng(1000 + n_kv + bs)
    k_tok = random_f16(rng, (max(n_kv, 1), G, D))
    got = oracle.block_keys(k_tok, n_kv, bs)
    assert np.array_equal(got, _keys_fraction(k_tok, n_kv, bs))


def test_block_keys_dyadic_blocks_vs_numpy():
    """Full blocks of 64 tokens: the sum of 64 fp16 values and its division
    by 64 are exact in float64, so numpy's float64 -> float16 conversion
    (correctly rounded) gives the fp16 mean."""
    rng = np.random.default_rng(31)
    n_kv, bs, G, D = 64 * 20, 64, 3, 128
    k_tok = qi.f64_to_f16_bits(rng.standard_normal((n_kv, G, D)) / math.sqrt(D))
    got = oracle.block_keys(k_tok, n_kv, bs)
    vals = k_tok.view(np.float16).astype(np.float64).reshape(n_kv // bs, bs, G, D)
    want = (vals.sum(axis=1) / bs).astype(np.float16).view(np.uint16).transpose(1, 0, 2)
    assert np.array_equal(got, want)


def test_block_keys_closed_forms():
    rng = np.random.default_rng(32)
    G, D, bs, nb = 2, 16, 8, 5
    # a block of one repeated key averages to that key; the partial last
    # block (3 tokens) to its own tokens' mean, not divided by bs
    key = random_f16(rng, (G, nb, D), special_frac=0.0)
    k_tok = np.repeat(key, bs, axis=1).transpose(1, 0, 2)[: (nb - 1) * bs + 3].copy()
    got = oracle.block_keys(k_tok, (nb - 1) * bs + 3, bs)
    assert np.array_equal(got, key)
    # integers: mean of 1..8 = 4.5; of (2, 4, 9) = 5; a zero mean is +0
    ints = np.zeros((11, 1, 2))
    ints[:8, 0, 0] = np.arange(1, 9)
    ints[8:, 0, 0] = [2, 4, 9]
    ints[:, 0, 1] = [1, -1] * 5 + [0]
    got = oracle.block_keys(qi.f64_to_f16_bits(ints), 11, 8)
    assert got[0, :, 0].view(np.float16).tolist() == [4.5, 5.0]
    assert got[0, :, 1].tolist() == [0, 0]


# --------------------------------------------------------------------------
# attention over the selected blocks (the step after the selection)
# --------------------------------------------------------------------------

def _attn_case(seed, nq=5, G=2, H=3, D=64, n_kv=64 * 6 + 9, bs=64, k=4, scale_v=1.0):
    rng = np.random.default_rng(seed)
    q16 = qi.f64_to_f16_bits(rng.standard_normal((nq, G, H, D)) * 0.5)
    kt = qi.f64_to_f16_bits(rng.standard_normal((n_kv, G, D)) * 0.5)
    vt = qi.f64_to_f16_bits(rng.standard_normal((n_kv, G, D)) * scale_v)
    nb = -(-n_kv // bs)
    ids = np.full((G, nq, k), -1, np.int32)
    for g in range(G):
        for t in range(nq):
            sel = rng.permutation(nb)[:min(k, nb)]
            ids[g, t, :sel.size] = sel
            if t == 1:
                ids[g, t, 1] = -1           # an empty slot in the middle
    return q16, kt, vt, ids, n_kv, bs


def _numpy_attention(q16, kt, vt, ids, n_kv, bs):
    """Dense float64 attention with numpy over an explicit token list."""
    nq, G, H, D = q16.shape
    Q = q16.view(np.float16).astype(np.float64)
    K = kt.view(np.float16).astype(np.float64)
    V = vt.view(np.float16).astype(np.float64)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    out = np.zeros((nq, G, H, D))
    for g in range(G):
        for t in range(nq):
            toks = [j for b in ids[g, t] if b >= 0 for j in range(b * bs, min((b + 1) * bs, n_kv))]
            if not toks:
                continue
            s = Q[t, g] @ K[toks, g].T * scale          # [H, L]
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[t, g] = (p @ V[toks, g]) / p.sum(axis=1, keepdims=True)
    return out


def test_attention_vs_numpy_dense():
    case = _attn_case(41)
    out, B = oracle.attention(*case)
    want = _numpy_attention(*case)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-14)
    assert np.all(B > 0)


def test_attention_closed_forms():
    q16, kt, vt, ids, n_kv, bs = _attn_case(42)
    # one selected token (a one-token tail block): the output is that value row
    n1 = 64 * 3 + 1
    one = np.full_like(ids, -1)
    one[:, :, 0] = 3                      # the tail block holds only token 192
    out, _ = oracle.attention(q16, kt[:n1], vt[:n1], one, n1, bs)
    V = vt.view(np.float16).astype(np.float64)
    for g in range(ids.shape[0]):
        assert np.array_equal(out[:, g], np.broadcast_to(V[192, g], out[:, g].shape))
    # zero queries: equal weights, the output is the mean of the selected values
    out, _ = oracle.attention(np.zeros_like(q16), kt, vt, ids, n_kv, bs)
    for g in range(ids.shape[0]):
        for t in range(q16.shape[0]):
            toks = [j for b in ids[g, t] if b >= 0 for j in range(b * bs, min((b + 1) * bs, n_kv))]
            assert np.allclose(out[t, g], V[toks, g].mean(axis=0), rtol=1e-12, atol=1e-15)
    # no selected block: zeros
    out, B = oracle.attention(q16, kt, vt, np.full_like(ids, -1), n_kv, bs)
    assert np.all(out == 0) and np.all(B == 0)


def test_attention_invariants():
    q16, kt, vt, ids, n_kv, bs = _attn_case(43)
    out, _ = oracle.attention(q16, kt, vt, ids, n_kv, bs)
    # the order of the selected ids does not matter
    perm = ids[:, :, ::-1].copy()
    outp, _ = oracle.attention(q16, kt, vt, perm, n_kv, bs)
    assert np.allclose(outp, out, rtol=1e-13, atol=1e-15)
    # values x2 -> output x2 exactly (every operation scales exactly)
    v2 = qi.f64_to_f16_bits(vt.view(np.float16).astype(np.float64) * 2)
    out2, _ = oracle.attention(q16, kt, v2, ids, n_kv, bs)
    assert np.array_equal(out2, out * 2)


def _fp32_device_model(q16, kt, vt, ids, n_kv, bs, no_rescale=False, drop_last=False,
                       scale_1_over_d=False, split_weights=False, no_unscale=False):
    """The device's algorithm in numpy float32: per row and head, chunks of
    up to 64 tokens in id order, a running maximum, chunk sums of P*V and P
    added into rescaled running sums.  split_weights: P*V from the weights'
    two fp16 parts scaled by 2^14 (hi = fp16(p*2^14), lo = fp16(p*2^14 -
    hi)), each part's products and sums in float32 of their own, the two
    added and unscaled at the end."""
    nq, G, H, D = q16.shape
    Q = q16.view(np.float16).astype(np.float32)
    K = kt.view(np.float16).astype(np.float32)
    V = vt.view(np.float16).astype(np.float32)
    scale = np.float32(1.0 / D if scale_1_over_d else 1.0 / math.sqrt(D))
    out = np.zeros((nq, G, H, D), np.float32)
    for g in range(G):
        for t in range(nq):
            toks = [j for b in ids[g, t] if b >= 0 for j in range(b * bs, min((b + 1) * bs, n_kv))]
            if drop_last:
                toks = toks[:-1]
            if not toks:
                continue
            m = np.full(H, -np.inf, np.float32)
            acc = np.zeros((H, D), np.float32)
            acc_lo = np.zeros((H, D), np.float32)
            den = np.zeros(H, np.float32)
            for c0 in range(0, len(toks), 64):
                ch = toks[c0:c0 + 64]
                s = np.einsum("hi,ji->hj", Q[t, g], K[ch, g]).astype(np.float32) * scale
                mn = np.maximum(m, s.max(axis=1))
                a = np.exp((m - mn).astype(np.float32)).astype(np.float32)
                p = np.exp((s - mn[:, None]).astype(np.float32)).astype(np.float32)
                if no_rescale:   # the running sums kept at the old maximum's scale
                    a = np.ones_like(a)
                if split_weights:
                    p14 = (p * np.float32(16384)).astype(np.float32)
                    hi = p14.astype(np.float16).astype(np.float32)
                    lo = (p14 - hi).astype(np.float16).astype(np.float32)
                    acc = acc * a[:, None] + (hi @ V[ch, g]).astype(np.float32)
                    acc_lo = acc_lo * a[:, None] + (lo @ V[ch, g]).astype(np.float32)
                else:
                    acc = acc * a[:, None] + (p @ V[ch, g]).astype(np.float32)
                den = den * a + p.sum(axis=1, dtype=np.float32)
                m = mn
            if split_weights:
                acc = (acc + acc_lo).astype(np.float32)
                if not no_unscale:
                    acc = (acc * np.float32(1.0 / 16384)).astype(np.float32)
            out[t, g] = acc / den[:, None]
    return out


def test_attention_bound_admits_fp32_model_and_rejects_mistakes():
    case = _attn_case(44, nq=4, G=2, H=4, D=128, n_kv=64 * 40 + 17, k=24)
    ref, B = oracle.attention(*case)
    good = _fp32_device_model(*case)
    res = oracle.check_attention(good, ref, B)
    assert res.ok, str(res)
    # the weighted values from the weights' two fp16 parts (the matrix-core
    # form) are within the same bound
    split = _fp32_device_model(*case, split_weights=True)
    res = oracle.check_attention(split, ref, B)
    assert res.ok, str(res)
    # and leaving the parts' 2^14 scale in is caught
    scaled = _fp32_device_model(*case, split_weights=True, no_unscale=True)
    assert not oracle.check_attention(scaled, ref, B).ok
    for kw in (dict(no_rescale=True), dict(drop_last=True), dict(scale_1_over_d=True)):
        bad = _fp32_device_model(*case, **kw)
        assert not oracle.check_attention(bad, ref, B).ok, kw
    assert not oracle.check_attention(ref + 2.5 * B, ref, B).ok


# ---------------------------------------------------------------------------
# The forced-tail rule (reading taken of the "+1e9 dead-tail rule", Strata
# pull request #856, "What": the partial last block gets 1e9 added to its
# score after the head sum).  Pinned by closed forms of fp32 and float64
# addition, by the ranking it must produce, and by the bound staying valid for
# the one extra fp32 rounding a device makes.
# ---------------------------------------------------------------------------

def pin_force_tail(force_fn, model_fn) -> None:
    cfg = qi.TINY                       # 15 full blocks and a 40-token tail block
    w = qi.make(cfg, with_q32=False)
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    fr = force_fn(ref, cfg.n_kv, cfg.bs)
    nf = cfg.nf
    # only the tail column moves, by 1e9 (f64: the scores are far below 2^29,
    # so s + 1e9 is exact to 2^-23 and equal to the sum of the two)
    assert np.array_equal(fr.score[:, :nf], ref.score[:, :nf])
    assert np.array_equal(fr.S, ref.S)
    assert np.array_equal(fr.B[:, :nf], ref.B[:, :nf])
    d = fr.score[:, nf] - ref.score[:, nf]
    assert np.all(np.abs(d - 1e9) <= 2.0 ** -22), d
    # the tail ranks first in every row, the other k - 1 slots as before
    ids_f = oracle.topk(fr.score, cfg.k)[0]
    ids_0 = oracle.topk(ref.score[:, :nf], cfg.k - 1)[0]
    assert np.all(ids_f[:, 0] == nf)
    assert np.array_equal(ids_f[:, 1:], ids_0)
    # the fixed-order fp32 model with the rule: fp32 spacing at 1e9 is 64 and
    # 1e9 is exact in fp32, so fl32(s + 1e9) = 1e9 + 64 * rne(s / 64) while s
    # stays far below 2^30 - 1e9
    m0 = model_fn(w.q16, w.kblk, nf, force_tail=False).astype(np.float64)
    m1 = model_fn(w.q16, w.kblk, nf, force_tail=True).astype(np.float64)
    assert np.all(m0 < 1e6)
    assert np.array_equal(m1, 1e9 + 64.0 * np.round(m0 / 64.0))
    # and it lies within the rule's bound of the exact forced score
    s_dev = ref.score.copy()
    s_dev[:, nf] = m1
    assert oracle.check_scores(s_dev, fr).ok
    # no partial block (the full blocks alone, n_kv = nf * bs): nothing changes
    r2 = oracle.Scores(ref.score[:, :nf], ref.S[:, :nf], ref.B[:, :nf], ref.rows)
    f2 = force_fn(r2, nf * cfg.bs, cfg.bs)
    assert np.array_equal(f2.score, r2.score) and np.array_equal(f2.B, r2.B)


def test_force_tail_rule():
    pin_force_tail(oracle.force_tail, oracle.block_model_f32)


def test_force_tail_bound_covers_fp32_rounding():
    """For any exact score s >= 0 of fp32 magnitude and any device value x
    within the unforced bound B0 of s, fl32(x + 1e9) is within the forced
    bound of s + 1e9: the rule's term 8*2^-24*1e9 (about 477) exceeds half
    the fp32 spacing at and above 1e9 (32 or 64) with room to spare."""
    rng = np.random.default_rng(11)
    s = np.concatenate([rng.random(20000) * 10.0 ** rng.integers(-3, 8, 20000),
                        [0.0, 31.9, 32.0, 32.1, 95.99, 96.0, 7.3e7]])
    S = s * (1.0 + rng.random(s.size) * 5.0)
    B0 = 2.0 ** -9.5 * S + 8.0 * 2.0 ** -24 * s
    x = (s + (rng.random(s.size) * 2.0 - 1.0) * B0).astype(np.float32)   # a device score
    forced = (x + np.float32(1e9)).astype(np.float64)
    exact = s + 1e9
    B1 = 2.0 ** -9.5 * S + 8.0 * 2.0 ** -24 * exact
    assert np.all(np.abs(forced - exact) <= B1)


@pytest.mark.parametrize("mutant", ["wrong_column", "bound_not_recomputed", "add_1e8",
                                    "model_adds_twice"])
def test_force_tail_pins_catch_planted_mistakes(mutant):
    def bad_force(ref, n_kv, bs):
        nf, nb = n_kv // bs, -(-n_kv // bs)
        if nb == nf:
            return ref
        col = nf - 1 if mutant == "wrong_column" else nf
        add = 1e8 if mutant == "add_1e8" else 1e9
        score, B = ref.score.copy(), ref.B.copy()
        score[:, col] += add
        if mutant != "bound_not_recomputed":
            B[:, col] = 2.0 ** -9.5 * ref.S[:, col] + 8.0 * 2.0 ** -24 * np.abs(score[:, col])
        return oracle.Scores(score, ref.S, B, ref.rows)

    def bad_model(q16, kblk, b, rows=None, force_tail=False):
        out = oracle.block_model_f32(q16, kblk, b, rows, force_tail)
        if force_tail and mutant == "model_adds_twice":
            out = (out + np.float32(1e9)).astype(np.float32)
        return out

    with pytest.raises(AssertionError):
        pin_force_tail(bad_force if mutant != "model_adds_twice" else oracle.force_tail,
                       bad_model)
