"""CPU check of the streaming selection's rules (the running per-row
candidate buffer of QSA_STREAM_SELECT, described in csrc/qsa_stream_row.h),
independent of the GPU: a plain model of those rules, applied to rows
streamed in 32-block tiles, must select exactly what a full sort selects --
the first min(k, nb) blocks by (score descending, block id ascending), NaN
last -- whatever the order, ties or NaNs of the scores.

The model follows the rules as stated, in float32 and 32-bit keys like the
device: admission when !(x < threshold) (NaN always admitted), a buffer of
128 entries in block-id order, compaction of a full row by a bisection on
16 leading key bits, or on all 32 with ties cut in buffer order when that
frees too little, and the final sort by (key descending, position ascending).
The reference is numpy's lexsort of the whole row.  Mutations of the rules
(an exact cut that skips the next key, a 16-bit cut that drops equal keys,
ties cut in the wrong order, NaN refused) are run too and must fail, so the
cases here can tell a wrong rule from a right one.  (Admitting keys equal to
the cut after an exact cut is not among them: that only admits more.)"""
from __future__ import annotations

import numpy as np
import pytest

CAP = 128
TILE = 32


def order_key(x: np.ndarray) -> np.ndarray:
    """32-bit order key of float32 scores (larger = better): NaN -> 0, -0 ->
    +0, then the sign-magnitude flip."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = np.where(u == 0x80000000, 0, u)
    k = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)
    k = np.where((u & 0x7FFFFFFF) > 0x7F800000, 0, k)
    return k.astype(np.uint64)


def admit_floor(adm: int) -> np.float32:
    if adm <= 0x80000000:
        return np.float32(-np.inf)
    b = min(adm - 0x80000000, 0x7F800000)
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def compact(vals, ids, kk, mut=None):
    """One row's compaction: returns the kept (vals, ids) in buffer order and
    the new admission key."""
    keys = order_key(np.array(vals, dtype=np.float32))

    def count_ge(t):
        return int((keys >= t).sum())

    T = 0
    for bit in range(31, 15, -1):
        if count_ge(T | (1 << bit)) >= kk:
            T |= 1 << bit
    keep = keys >= T
    if mut == "16bit_gt":
        keep = keys > T
    adm = T
    if T == 0 or keep.sum() > CAP - TILE:
        for bit in range(15, -1, -1):
            if count_ge(T | (1 << bit)) >= kk:
                T |= 1 << bit
        gt = keys > T
        need = kk - int(gt.sum())
        eq_pos = np.flatnonzero(keys == T)
        if mut == "ties_last":
            eq_pos = eq_pos[::-1]
        take = np.zeros_like(gt)
        take[eq_pos[:need]] = True
        keep = gt | take
        adm = T + 2 if mut == "exact_skips_next_key" else T + 1
    return [v for v, k in zip(vals, keep) if k], [i for i, k in zip(ids, keep) if k], adm


def admitted(x, th, mut) -> bool:
    if mut == "nan_refused":
        return bool(x >= th)
    return not (x < th)   # NaN admitted


def stream_select(x: np.ndarray, k: int, mut=None, eager=0.0, rng=None):
    """The streaming rules on one row x (float32, block order).  eager: the
    chance that a row more than 88 full is compacted early (the device does
    so when another row of the wave needs a compaction)."""
    nb = len(x)
    kk = min(k, nb)
    vals, ids, adm = [], [], 0
    for t0 in range(0, nb, TILE):
        th = admit_floor(adm)
        tile = range(t0, min(nb, t0 + TILE))
        cand = [b for b in tile if admitted(x[b], th, mut)]
        if len(vals) + len(cand) > CAP or (eager and len(vals) > CAP - 40 and rng.random() < eager):
            vals, ids, adm = compact(vals, ids, kk, mut)
            th = admit_floor(adm)
            cand = [b for b in tile if admitted(x[b], th, mut)]
        assert len(vals) + len(cand) <= CAP
        vals += [x[b] for b in cand]
        ids += cand
    keys = order_key(np.array(vals, dtype=np.float32))
    order = np.lexsort((np.arange(len(vals)), -keys.astype(np.float64)))
    return [ids[i] for i in order[:kk]]


def exact_select(x: np.ndarray, k: int):
    keys = order_key(x)
    order = np.lexsort((np.arange(len(x)), -keys.astype(np.float64)))
    return [int(i) for i in order[: min(k, len(x))]]


def rows():
    rng = np.random.default_rng(7)
    out = []
    for nb in (50, 128, 129, 700, 2049):
        out.append((f"normal_nb{nb}", np.abs(rng.standard_normal(nb)).astype(np.float32)))
    n = 2049
    out.append(("rising", np.linspace(1, 2, n).astype(np.float32)))
    out.append(("falling", np.linspace(2, 1, n).astype(np.float32)))
    out.append(("sawtooth", np.tile(np.linspace(1, 2, 97), 22)[:n].astype(np.float32)))
    out.append(("few_values", rng.integers(0, 5, n).astype(np.float32)))
    out.append(("binary", (rng.random(n) < 0.05).astype(np.float32)))
    out.append(("all_zero", np.zeros(n, np.float32)))
    out.append(("all_equal", np.full(n, 3.5, np.float32)))
    near = (1 + rng.integers(0, 3, n) * 2.0 ** -23).astype(np.float32)   # one-ulp ties
    out.append(("ulp_ties", near))
    nan = np.abs(rng.standard_normal(n)).astype(np.float32)
    nan[rng.random(n) < 0.3] = np.nan
    out.append(("nan30", nan))
    allnan = np.full(n, np.nan, np.float32)
    allnan[rng.integers(0, n, 20)] = 1.0
    out.append(("nan_mostly", allnan))
    inf = np.abs(rng.standard_normal(n)).astype(np.float32)
    inf[::50] = np.inf
    out.append(("inf_every50", inf))
    return out


ROWS = rows()


@pytest.mark.parametrize("k", [1, 7, 64])
@pytest.mark.parametrize("name,x", ROWS, ids=[r[0] for r in ROWS])
def test_stream_rules_select_exactly(name, x, k):
    want = exact_select(x, k)
    assert stream_select(x, k) == want
    # early compactions (another row of the wave triggered one) change nothing
    assert stream_select(x, k, eager=0.5, rng=np.random.default_rng(3)) == want


@pytest.mark.parametrize("mut", ["exact_skips_next_key", "16bit_gt", "ties_last", "nan_refused"])
def test_stream_rule_mutations_fail(mut):
    """Each mutated rule gives a wrong selection on at least one of the rows."""
    wrong = 0
    for _, x in ROWS:
        for k in (7, 64):
            if stream_select(x, k, mut=mut) != exact_select(x, k):
                wrong += 1
    assert wrong > 0, f"mutation {mut} not detected"
