"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Bars (contract of Strata pull request #228, part 1, and pull request #856):
  * every score within B = 2^-9.5*S + 8*2^-24*|score_ref| of the oracle;
    +2.5*B perturbations of the same scores must fail the same check;
  * the tail block bit for bit equal to the oracle's fixed-order fp32 model;
  * ids bit for bit equal to the oracle's top-k of the device's own scores,
    and equal to the oracle's selection except near-ties within 2*B;
  * zero tolerance on the coordinate-coded and integer fixtures;
  * exact write sets (canaries), bitwise determinism across launches,
    exactly 64x scores for x8 inputs.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
from gpu_util import (SENTINEL, dev, guarded, k_dev, log, q_dev, run_block_scores,
                      scores_mask)

pytestmark = pytest.mark.gpu

import sparse_attention_block_qsa_amd as qsa  # noqa: E402  (fails loudly if not built)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check_bound(s_gpu, ref, name, exact=False):
    res = oracle.check_scores(s_gpu, ref)
    log(f"  [{name}] {res}")
    assert res.ok, f"{name}: {res}"
    if exact:
        assert np.array_equal(s_gpu, ref.score), f"{name}: not exact"
    f1, f2 = oracle.negative_controls(ref, s_gpu)
    assert f1 and f2, f"{name}: negative control passed the checker"
    return res


def check_ids(ids_gpu, s_gpu, ref, k, name):
    want = oracle.topk(s_gpu, k)[0]
    assert np.array_equal(ids_gpu, want), f"{name}: ids differ from the top-k of the device scores"
    sel = oracle.check_selection(ids_gpu, ref, k)
    log(f"  [{name}] selection: rows differing {sel.rows_differing}, ids differing "
        f"{sel.ids_differing}/{sel.n_ids}, worst gap/2B {sel.worst_gap_ratio:.3f}")
    assert sel.ok, f"{name}: {sel.detail}"


def run_topk_dev(s_rows: np.ndarray, nb: int, k: int, ld_pad: int = 5, want_vals=True):
    rows = s_rows.shape[0]
    ld = max(nb, 1) + ld_pad
    src = torch.full((rows, ld), float("nan"), dtype=torch.float32, device=dev())
    if nb:
        src[:, :nb] = torch.from_numpy(np.ascontiguousarray(s_rows, dtype=np.float32)).to(dev())
    ids = guarded((rows, k + 2), torch.int32)
    vals = guarded((rows, k + 2), torch.float32) if want_vals else None
    qsa.select_topk(src, nb, k, ids=ids.view, vals=vals.view if vals else None)
    torch.cuda.synchronize()
    m = np.zeros((rows, k + 2), dtype=bool)
    m[:, :k] = True
    assert ids.outside_intact(m) and ids.written_all(m), "select_topk ids write set"
    if vals:
        assert vals.outside_intact(m) and vals.written_all(m), "select_topk vals write set"
    out_ids = ids.view[:, :k].cpu().numpy()
    out_vals = vals.view[:, :k].cpu().numpy() if vals else None
    return out_ids, out_vals


# ---------------------------------------------------------------------------
# conversion
# ---------------------------------------------------------------------------

def test_convert_all_fp32_patterns():
    """The conversion kernel equals the oracle's round-to-nearest-even on
    every one of the 2^32 fp32 bit patterns (NaN payload rule included)."""
    chunk = 1 << 26
    n_bad = 0
    for c in range((1 << 32) // chunk):
        start = c * chunk
        pat = (torch.arange(start, start + chunk, dtype=torch.int64, device=dev())
               & 0xFFFFFFFF).to(torch.int32).view(torch.float32)
        out = qsa.convert_f32_f16(pat)
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        want = oracle.convert_f32_f16(qi.fp32_bit_patterns(start, chunk))
        bad = np.flatnonzero(got != want)
        n_bad += bad.size
        if bad.size:
            i = int(bad[0])
            log(f"  chunk {c}: {bad.size} mismatches, first {start + i:#010x}: "
                f"got {got[i]:#06x} want {want[i]:#06x}")
        if c % 16 == 15:
            log(f"  convert: {c + 1} / 64 chunks checked")
    assert n_bad == 0


@pytest.mark.parametrize("n,off_src,off_dst", [(1, 0, 0), (7, 0, 0), (8, 0, 0), (4099, 0, 0),
                                               (1000, 1, 0), (1000, 0, 1), (1000, 3, 5)])
def test_convert_lengths_and_alignment(n, off_src, off_dst):
    x = qi.normal(77, 1, n + off_src).astype(np.float32) * 1000
    src = torch.from_numpy(x).to(dev())[off_src:off_src + n]
    buf = torch.full((n + off_dst + 8,), 0x5A5A, dtype=torch.int16, device=dev())
    dst = buf[off_dst:off_dst + n]
    st = qsa.lib.qsa_convert_f32_f16(qsa._ptr(src), qsa._ptr(dst), n, qsa._stream(None))
    assert st == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.convert_f32_f16(x[off_src:off_src + n]))
    rest = buf.cpu().numpy()
    assert np.all(rest[:off_dst] == 0x5A5A) and np.all(rest[off_dst + n:] == 0x5A5A)


# ---------------------------------------------------------------------------
# scores on the configs
# ---------------------------------------------------------------------------

SMALL = ["tiny_nq37_nkv1000", "nq256_nkv4096", "nq256_nkv32768", "nq256_nkv131072"]


@pytest.mark.parametrize("name", SMALL)
def test_config_scores_ids_and_write_set(name):
    cfg = qi.CONFIGS[name]
    log(f"config {name}")
    w = qi.make(cfg)
    s_gpu, intact, written = run_block_scores(w.q16, w.kblk, cfg.n_kv, cfg.bs)
    assert intact, "scores: write outside [r][0, nb)"
    assert written, "scores: a cell of [r][0, nb) was not written"
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    check_bound(s_gpu, ref, name)
    if cfg.nb > cfg.nf:   # tail block: bit for bit the fixed-order model
        model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
        assert np.array_equal(s_gpu[:, cfg.nf].astype(np.float32).view(np.uint32),
                              model.view(np.uint32)), "tail block differs from the model"
    ids, vals = run_topk_dev(s_gpu, cfg.nb, cfg.k)
    check_ids(ids, s_gpu, ref, cfg.k, name)
    sel = ids >= 0
    assert np.array_equal(vals[sel], s_gpu[np.nonzero(sel)[0], ids[sel]].astype(np.float32))
    # determinism: a second launch is bitwise identical
    s2, _, _ = run_block_scores(w.q16, w.kblk, cfg.n_kv, cfg.bs)
    assert np.array_equal(s_gpu.view(np.uint64), s2.view(np.uint64)), "not deterministic"


# decode shapes: few queries per KV head (G, nq, H, D, n_kv, k)
DECODE_SHAPES = [
    (8, 1, 8, 128, 131109, 64),    # the bench's decode step: 2049 blocks, 37-token tail
    (8, 4, 8, 128, 20 * 64, 64),   # k > nb/2, no tail
    (2, 3, 16, 64, 5000, 16),      # H = 16: two queries x 16 heads per MFMA row block
    (4, 8, 4, 64, 3 * 64 + 63, 8), # H = 4, three full blocks and a 63-token tail
    (3, 2, 5, 128, 40, 4),         # a single partial block (no full block)
    (8, 1, 8, 128, (1 << 20) + 41, 64),   # a 1M-token decode step: 16385 blocks, rows past 4096 blocks
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda v: "G{}_nq{}_H{}_D{}_nkv{}_k{}".format(*v))
def test_decode_shapes_phase(shape):
    """One decode step per KV head through the whole phase (fp32 queries,
    conversion, the small scorer with the tail block, top-k): scores within
    the bound, the tail bit for bit the fixed-order model, ids exactly the
    top-k of the device scores and near-tie consistent with the oracle's."""
    G, nq, H, D, n_kv, k = shape
    cfg = qi.Config("decode", G, nq, H, D, n_kv, 64, k, "normal", 7000 + G * 10 + nq)
    log(f"decode {shape}")
    w = qi.make(cfg)
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                            with_vals=True)
    ids, vals = qsa.select_phase(torch.from_numpy(w.q32).to(dev()), k_dev(w.kblk), cfg.n_kv,
                                 cfg.bs, cfg.k, ws)
    torch.cuda.synchronize()
    s_gpu = ws.scores[:, :, :cfg.nb].reshape(cfg.rows, cfg.nb).cpu().numpy().astype(np.float64)
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    check_bound(s_gpu, ref, "decode")
    if cfg.nb > cfg.nf:
        model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
        assert np.array_equal(s_gpu[:, cfg.nf].astype(np.float32).view(np.uint32),
                              model.view(np.uint32))
    got = ids.reshape(cfg.rows, cfg.k).cpu().numpy()
    check_ids(got, s_gpu, ref, cfg.k, "decode")
    sel = got >= 0
    v = vals.reshape(cfg.rows, cfg.k).cpu().numpy()
    assert np.array_equal(v[sel], s_gpu[np.nonzero(sel)[0], got[sel]].astype(np.float32))
    assert np.all(v[~sel] == -np.inf)


def _random_phase_case(i):
    """Case i of the seeded randomised phase sweep: KV heads, queries, heads,
    head dim, block size, context length, k and a query chunk; every twelfth
    case has enough query rows for the wide scorer."""
    rng = np.random.default_rng(9000 + i)
    if i % 12 == 11:
        G, nq = 4, 4096 + int(rng.integers(0, 64))
        H = int(rng.choice([4, 8, 12]))
        D = 64 if H == 12 else 128
        bs = 64
        n_kv = int(rng.integers(1, 12)) * bs + int(rng.integers(0, bs))
    else:
        G = int(rng.choice([1, 2, 3, 4, 8]))
        nq = int(rng.integers(1, 400))
        H = int(rng.integers(1, 17))
        D = int(rng.choice([64, 128]))
        bs = int(rng.choice([8, 16, 32, 64, 128]))
        n_kv = int(rng.integers(0, 3000))
    k = int(rng.integers(1, 65))
    q_chunk = 0 if i % 3 else int(rng.integers(1, nq + 1))
    return G, nq, H, D, n_kv, bs, k, q_chunk


@pytest.mark.parametrize("i", range(24))
def test_phase_randomised_geometry(i):
    """Seeded random geometries through the whole phase with fp32 queries:
    scores within the bound, the tail bit for bit the fixed-order model, ids
    the top-k of the device scores and near-tie consistent with the oracle's,
    values bit for bit; with a query chunk, the same bits as one pass."""
    G, nq, H, D, n_kv, bs, k, q_chunk = _random_phase_case(i)
    log(f"phase case {i}: G {G} nq {nq} H {H} D {D} n_kv {n_kv} bs {bs} k {k} q_chunk {q_chunk}")
    cfg = qi.Config("rphase", G, nq, H, D, n_kv, bs, k, "normal", 9100 + i)
    w = qi.make(cfg)
    q = torch.from_numpy(w.q32).to(dev())
    kb = k_dev(w.kblk)

    def run(chunk):
        ws = qsa.PhaseWorkspace(nq, G, H, D, n_kv, bs, k, dev(), with_vals=True, q_chunk=chunk)
        ids, vals = qsa.select_phase(q, kb, n_kv, bs, k, ws)
        torch.cuda.synchronize()
        return ws, ids.reshape(cfg.rows, k).cpu().numpy(), vals.reshape(cfg.rows, k).cpu().numpy()

    # one pass over every query: all scores stay in the workspace
    ws, got, v = run(0)
    nb = cfg.nb
    if nb == 0:
        assert np.all(got == -1) and np.all(v == -np.inf)
        return
    s_gpu = ws.scores[:, :, :nb].reshape(cfg.rows, nb).cpu().numpy().astype(np.float64)
    ref = oracle.scores(w.q16, w.kblk, nb)
    check_bound(s_gpu, ref, "rphase")
    if nb > cfg.nf:
        model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
        assert np.array_equal(s_gpu[:, cfg.nf].astype(np.float32).view(np.uint32),
                              model.view(np.uint32))
    check_ids(got, s_gpu, ref, k, "rphase")
    sel = got >= 0
    assert np.array_equal(v[sel].view(np.uint32),
                          s_gpu[np.nonzero(sel)[0], got[sel]].astype(np.float32).view(np.uint32))
    assert np.all(v[~sel] == -np.inf)
    if q_chunk:
        # the host walks the queries in chunks of q_chunk through a workspace
        # of G*qc rows: ids and values bit for bit those of one pass, and the
        # workspace holds the last chunk's scores (query t0 + t' of KV head g
        # at row g*n + t')
        wsc, gotc, vc = run(q_chunk)
        qc = wsc.chunk_rows
        assert qc == min(q_chunk, nq) and wsc.scores.shape[1] == qc
        assert np.array_equal(gotc, got)
        assert np.array_equal(vc.view(np.uint32), v.view(np.uint32))
        t0 = ((nq - 1) // qc) * qc
        n = nq - t0
        last = wsc.scores.reshape(-1, wsc.ld_s)[:G * n].reshape(G, n, wsc.ld_s)[:, :, :nb]
        assert torch.equal(last.view(torch.int32), ws.scores[:, t0:, :nb].view(torch.int32))


def test_tiny_nkv0_writes_nothing_and_selects_nothing():
    cfg = qi.TINY
    w = qi.make(cfg)
    out = guarded((cfg.G, cfg.nq, 8), torch.float32)
    qsa.block_scores(q_dev(w.q16), k_dev(w.kblk), 0, cfg.bs, out=out.view)
    torch.cuda.synchronize()
    assert out.outside_intact(np.zeros((cfg.G, cfg.nq, 8), dtype=bool))
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, 0, cfg.bs, cfg.k, dev(), with_vals=True)
    ws.ids.fill_(123)
    ids, vals = qsa.select_phase(torch.from_numpy(w.q32).to(dev()), k_dev(w.kblk), 0, cfg.bs,
                                 cfg.k, ws)
    torch.cuda.synchronize()
    assert torch.all(ids == -1) and torch.all(vals == -float("inf"))


def test_coded_fixture_exact():
    cfg = qi.CONFIGS["nq256_nkv32768"]
    w = qi.coded_fixture(cfg)
    s_gpu, intact, written = run_block_scores(w.q16, w.kblk, cfg.n_kv, cfg.bs)
    assert intact and written
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    check_bound(s_gpu, ref, "coded", exact=True)
    ids, _ = run_topk_dev(s_gpu, cfg.nb, cfg.k)
    assert np.array_equal(ids, oracle.topk(ref.score, cfg.k)[0]), "coded: ids not exact"


@pytest.mark.parametrize("n_kv", [4096, 4096 + 37])
def test_integer_fixture_exact(n_kv):
    cfg = qi.CONFIGS["nq256_nkv4096"]
    cfg = qi.Config("int", cfg.G, cfg.nq, cfg.H, cfg.D, n_kv, cfg.bs, cfg.k, "normal", 0)
    w = qi.integer_fixture(cfg)
    s_gpu, intact, written = run_block_scores(w.q16, w.kblk, cfg.n_kv, cfg.bs)
    assert intact and written
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    check_bound(s_gpu, ref, f"integer n_kv={n_kv}", exact=True)
    ids, _ = run_topk_dev(s_gpu, cfg.nb, cfg.k)
    assert np.array_equal(ids, oracle.topk(ref.score, cfg.k)[0])


def test_x8_headroom_exactly_64x():
    cfg = qi.HEADLINE
    w = qi.make(cfg)
    w8 = qi.scaled_by_8(w)
    s1, _, _ = run_block_scores(w.q16, w.kblk, cfg.n_kv, cfg.bs)
    s8, intact, written = run_block_scores(w8.q16, w8.kblk, cfg.n_kv, cfg.bs)
    assert intact and written
    ref8 = oracle.scores(w8.q16, w8.kblk, cfg.nb)
    check_bound(s8, ref8, "x8")
    assert np.array_equal(s8, s1 * 64.0), "x8 inputs did not give exactly 64x scores"
    ids, _ = run_topk_dev(s8, cfg.nb, cfg.k)
    check_ids(ids, s8, ref8, cfg.k, "x8")


def test_stress60_within_bound():
    cfg = qi.CONFIGS["nq256_nkv4096"]
    cfg = qi.Config("stress60", 1, 64, 8, 128, 4096 + 19, 64, 16, "normal", 0)
    w = qi.stress60_fixture(cfg)
    s_gpu, intact, written = run_block_scores(w.q16, w.kblk, cfg.n_kv, cfg.bs)
    assert intact and written
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    check_bound(s_gpu, ref, "stress60")
    model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
    assert np.array_equal(s_gpu[:, cfg.nf].astype(np.float32).view(np.uint32),
                          model.view(np.uint32))


# ---------------------------------------------------------------------------
# ragged geometry, strides, head passes
# ---------------------------------------------------------------------------

GEOMS = [
    # G, nq, H, D, n_kv, bs, tok_pad, nb_pad
    (1, 1, 1, 64, 64, 64, 0, 0),
    (1, 15, 2, 64, 31 * 64, 64, 8, 1),
    (2, 17, 3, 128, 33 * 64 + 1, 64, 0, 2),
    (3, 65, 5, 64, 95 * 16 + 15, 16, 24, 0),
    (1, 100, 8, 128, 7, 64, 0, 0),           # only a tail block
    (2, 63, 9, 128, 40 * 32, 32, 8, 3),      # two head passes
    (1, 70, 12, 64, 65 * 64 + 63, 64, 0, 0),
    (1, 33, 16, 64, 20 * 64 + 9, 64, 16, 0), # D=64, two head passes
    (1, 50, 16, 128, 18 * 64, 64, 0, 1),     # D=128, two full passes
    (2, 129, 4, 128, 100 * 64 + 3, 64, 0, 0),
    # only a tail block (the standalone tail kernel): H = 16 and 5, D = 64,
    # one-token blocks, and more items than the kernel's grid (a second loop
    # trip per workgroup)
    (2, 300, 16, 64, 33, 64, 8, 0),
    (3, 129, 5, 128, 63, 64, 0, 1),
    (1, 1000, 1, 64, 1, 2, 0, 0),
    (4, 4200, 8, 128, 40, 64, 0, 0),
    # enough query rows (>= 256 groups of 64 over the KV heads) for the wide
    # scorer, which scores the tail block in the same launch
    (4, 4096, 8, 128, 40 * 64 + 5, 64, 0, 0),
    (2, 8192, 12, 64, 20 * 64 + 9, 64, 8, 1),     # two head passes, padded rows
    (4, 4100, 5, 128, 33 * 64, 64, 0, 0),         # ragged query groups, odd H
]


@pytest.mark.parametrize("geo", GEOMS, ids=lambda g: "G{}_nq{}_H{}_D{}_nkv{}_bs{}".format(*g[:6]))
def test_ragged_geometry(geo):
    G, nq, H, D, n_kv, bs, tok_pad, nb_pad = geo
    cfg = qi.Config("geo", G, nq, H, D, n_kv, bs, min(64, 8), "normal", 500 + nq)
    w = qi.make(cfg)
    s_gpu, intact, written = run_block_scores(w.q16, w.kblk, n_kv, bs, tok_pad=tok_pad,
                                              nb_pad=nb_pad)
    assert intact, "write outside the documented set"
    assert written, "a cell was not written"
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    check_bound(s_gpu, ref, "geo")
    if cfg.nb > cfg.nf:
        model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
        assert np.array_equal(s_gpu[:, cfg.nf].astype(np.float32).view(np.uint32),
                              model.view(np.uint32))


# ---------------------------------------------------------------------------
# top-k selector on identical inputs (bit exact)
# ---------------------------------------------------------------------------

def topk_cases():
    rng = np.random.default_rng(42)
    cases = []
    # 520, 1100, 3000: few-row selector shapes whose last waves hold few or none of the values
    for nb in (1, 5, 63, 64, 65, 200, 520, 1100, 2049, 3000, 4096, 5000):
        cases.append(("random", rng.standard_normal((13, nb)).astype(np.float32), nb))
    nb = 300
    cases.append(("all_equal", np.full((4, nb), 0.5, np.float32), nb))
    cases.append(("all_zero", np.zeros((4, nb), np.float32), nb))
    z = rng.integers(0, 2, (6, nb)).astype(np.float32) * 0.0
    z[rng.random((6, nb)) < 0.5] = -0.0
    cases.append(("signed_zeros", z, nb))
    d = rng.integers(-3, 3, (6, nb)).astype(np.float32)
    cases.append(("duplicates", d, nb))
    s = rng.standard_normal((6, nb)).astype(np.float32)
    s[rng.random((6, nb)) < 0.1] = np.nan
    s[rng.random((6, nb)) < 0.05] = np.inf
    s[rng.random((6, nb)) < 0.05] = -np.inf
    s[0, :] = np.nan
    cases.append(("nan_inf", s, nb))
    t = rng.standard_normal((4, 2049)).astype(np.float32)
    t[:, ::3] = 1.25
    cases.append(("many_ties_2049", t, 2049))
    # the sampled-threshold path with ties at the threshold: few distinct values
    q = (rng.integers(0, 1000, (8, 2049)) / 8.0).astype(np.float32)
    cases.append(("quantised_ties_2049", q, 2049))
    # +0 / -0 ties straddling the threshold, the rest negative
    zz = -1.0 - rng.random((6, 500)).astype(np.float32)
    for r in range(6):
        pos = rng.choice(500, 70, replace=False)
        zz[r, pos[:30]] = rng.random(30).astype(np.float32) + 1.0
        zz[r, pos[30:50]] = 0.0
        zz[r, pos[50:]] = -0.0
    cases.append(("signed_zero_threshold_500", zz, 500))
    # the same special values in rows of more than 512 blocks: the four-wave
    # few-row selector and, repeated, the 33-column many-rows one
    s2 = rng.standard_normal((6, 2049)).astype(np.float32)
    s2[rng.random((6, 2049)) < 0.1] = np.nan
    s2[rng.random((6, 2049)) < 0.03] = np.inf
    s2[rng.random((6, 2049)) < 0.03] = -np.inf
    s2[0, :] = np.nan
    s2[1, 40:] = np.nan   # fewer numbers than k: NaNs selected, in id order
    cases.append(("nan_inf", s2, 2049))
    z2 = -1.0 - rng.random((6, 1100)).astype(np.float32)
    for r in range(6):
        pos = rng.choice(1100, 70, replace=False)
        z2[r, pos[:30]] = rng.random(30).astype(np.float32) + 1.0
        z2[r, pos[30:50]] = 0.0
        z2[r, pos[50:]] = -0.0
    cases.append(("signed_zero_threshold_1100", z2, 1100))
    # Pairs of equal values inside the top 64 and one straddling the 64th
    # place, otherwise distinct values; and rows whose top values span many
    # binades (a few huge values among normal ones): the selector's sort of
    # 32-bit words must hand both kinds back to its sort of composites.
    for nbt in (300, 2049):
        pt = rng.standard_normal((6, nbt)).astype(np.float32)
        for r in range(6):
            order = np.argsort(-pt[r], kind="stable")
            for rank in (3, 20, 63):
                pt[r, order[rank + 1]] = pt[r, order[rank]]
        cases.append((f"paired_ties_{nbt}", pt, nbt))
        wr = rng.standard_normal((6, nbt)).astype(np.float32)
        for r in range(6):
            wr[r, rng.choice(nbt, 5, replace=False)] = np.float32(1e30) * rng.random(5).astype(np.float32)
        cases.append((f"wide_range_{nbt}", wr, nbt))
    # 150 tied maxima per row: more candidates than the few-row selector's
    # pooled path holds, so its per-wave selection and merges decide, ties
    # spread over the four waves' columns
    for nbt in (1100, 2049):
        tt = rng.standard_normal((4, nbt)).astype(np.float32)
        for r in range(4):
            tt[r, rng.choice(nbt, 150, replace=False)] = 3.0
        cases.append((f"tied_top_{nbt}", tt, nbt))
    cases.append(("all_negative_100", -rng.random((6, 100)).astype(np.float32) - 0.5, 100))
    # rows of at most 128 blocks, which are sorted whole (one or two
    # register columns): the special values and ties of the rows above
    for nbs in (50, 64, 100, 128):
        s3 = rng.standard_normal((6, nbs)).astype(np.float32)
        s3[rng.random((6, nbs)) < 0.15] = np.nan
        s3[rng.random((6, nbs)) < 0.05] = np.inf
        s3[rng.random((6, nbs)) < 0.05] = -np.inf
        s3[0, :] = np.nan
        s3[1, 10:] = np.nan   # fewer numbers than k: NaNs selected, in id order
        cases.append(("nan_inf", s3, nbs))
        z3 = rng.integers(-2, 3, (6, nbs)).astype(np.float32)
        z3[z3 == 0] = np.where(rng.random(int((z3 == 0).sum())) < 0.5, 0.0, -0.0)
        cases.append(("signed_zero_duplicates", z3, nbs))
    cases.append(("all_equal", np.full((4, 128), 0.5, np.float32), 128))
    cases.append(("all_zero", np.zeros((4, 100), np.float32), 100))
    cases.append(("all_negative_2049", -rng.random((4, 2049)).astype(np.float32), 2049))
    return cases


@pytest.mark.parametrize("case", topk_cases(), ids=lambda c: f"{c[0]}_nb{c[2]}")
@pytest.mark.parametrize("k", [1, 7, 64])
def test_topk_bit_exact(case, k):
    _, s, nb = case
    ids, vals = run_topk_dev(s, nb, k)
    want_ids, want_vals = oracle.topk(s.astype(np.float64), k)
    assert np.array_equal(ids, want_ids)
    sel = ids >= 0
    got_bits = vals[sel].view(np.uint32)
    want_bits = s[np.nonzero(sel)[0], ids[sel]].view(np.uint32)
    assert np.array_equal(got_bits, want_bits)
    assert np.all(vals[~sel] == -np.inf)


@pytest.mark.parametrize("case", topk_cases(), ids=lambda c: f"{c[0]}_nb{c[2]}")
def test_topk_many_rows_path_bit_exact(case):
    """The same rows repeated to 4096+ rows: the selector's many-rows launch
    (four rows per workgroup instead of one, candidates sorted as 32-bit
    words where exact): ids and values bit for bit the oracle's top-k for
    k = 64 and k = 5."""
    _, s, nb = case
    reps = -(-4096 // s.shape[0])
    big = np.ascontiguousarray(np.tile(s, (reps, 1)))
    for k in (64, 5):
        ids, vals = run_topk_dev(big, nb, k)
        want_ids, _ = oracle.topk(big.astype(np.float64), k)
        assert np.array_equal(ids, want_ids)
        sel = ids >= 0
        assert np.array_equal(vals[sel].view(np.uint32),
                              big[np.nonzero(sel)[0], ids[sel]].view(np.uint32))


def _long_topk_rows(nb, mix, rng):
    if mix == "normal":
        return rng.standard_normal((3, nb)).astype(np.float32)
    if mix == "quantised":   # few levels: long runs of ties straddle the k-th place
        return (rng.integers(0, 40, (3, nb)) / 4.0).astype(np.float32)
    if mix == "special":
        s = rng.standard_normal((3, nb)).astype(np.float32)
        s[rng.random((3, nb)) < 0.05] = np.nan
        s[rng.random((3, nb)) < 0.0002] = np.inf
        s[rng.random((3, nb)) < 0.01] = -np.inf
        return s
    return np.full((3, nb), -1.25, np.float32)   # all equal: the first k ids


@pytest.mark.parametrize("nb", [65536 + 37, 262144 + 3])
@pytest.mark.parametrize("mix", ["normal", "quantised", "special", "equal"])
def test_topk_long_rows(nb, mix):
    """Rows far past the selector's register-resident lengths (64 K and
    256 K blocks, ragged): ids and values bit for bit the oracle's top-k for
    k = 64 and k = 1."""
    rng = np.random.default_rng(nb + len(mix))
    s = _long_topk_rows(nb, mix, rng)
    log(f"long rows nb={nb} mix={mix}")
    for k in (64, 1):
        ids, vals = run_topk_dev(s, nb, k)
        want_ids, _ = oracle.topk(s.astype(np.float64), k)
        assert np.array_equal(ids, want_ids)
        sel = ids >= 0
        assert np.array_equal(vals[sel].view(np.uint32), s[np.nonzero(sel)[0], ids[sel]].view(np.uint32))


def _random_topk_case(i):
    """Case i of the seeded randomised selector sweep: a row length near one
    of the selector's boundaries, few or many rows, any k, and one of five
    value mixes (normal; quantised, many ties; NaN and infinities; a block
    of tied maxima; a few huge values among normal ones)."""
    rng = np.random.default_rng(7000 + i)
    ranges = [(1, 80), (500, 600), (1000, 1200), (2000, 2200), (3000, 4100), (4097, 6000),
              (60, 520), (2049, 2112)]
    lo, hi = ranges[i % 8]
    nb = int(rng.integers(lo, hi + 1))
    many = i % 8 == 7   # the many-rows launch at the prefill chunk's row length
    rows = 4096 + int(rng.integers(0, 64)) if many else int(rng.integers(1, 65))
    k = int(rng.integers(1, 65))
    mix = i % 5
    s = rng.standard_normal((rows, nb)).astype(np.float32)
    if mix == 1:
        s = (rng.integers(0, int(rng.integers(5, 2000)), (rows, nb)) / 8.0).astype(np.float32)
    elif mix == 2:
        s[rng.random((rows, nb)) < 0.08] = np.nan
        s[rng.random((rows, nb)) < 0.02] = np.inf
        s[rng.random((rows, nb)) < 0.02] = -np.inf
    elif mix == 3:
        n_tied = int(rng.integers(1, min(nb, 200) + 1))
        for r in range(rows):
            s[r, rng.choice(nb, n_tied, replace=False)] = 4.0
    elif mix == 4:
        s[rng.random((rows, nb)) < 0.003] = np.float32(3e28)
    return s, nb, k


@pytest.mark.parametrize("i", range(48))
def test_topk_randomised_shapes(i):
    """Seeded random selector cases across the launch forms (one wave per
    row, four rows per workgroup, four waves per row, the re-reading path):
    ids and values bit for bit the oracle's top-k of the same fp32 rows."""
    s, nb, k = _random_topk_case(i)
    print(f"case {i}: rows {s.shape[0]}, nb {nb}, k {k}", flush=True)
    ids, vals = run_topk_dev(s, nb, k)
    want_ids, _ = oracle.topk(s.astype(np.float64), k)
    assert np.array_equal(ids, want_ids), f"case {i}: rows {s.shape[0]}, nb {nb}, k {k}"
    sel = ids >= 0
    assert np.array_equal(vals[sel].view(np.uint32), s[np.nonzero(sel)[0], ids[sel]].view(np.uint32))
    assert np.all(vals[~sel] == -np.inf)


def test_topk_k_larger_than_nb_and_empty_rows():
    s = np.arange(10, dtype=np.float32)[None, :].repeat(3, 0)
    ids, vals = run_topk_dev(s, 10, 16)
    assert np.array_equal(ids[:, :10], np.tile(np.arange(9, -1, -1), (3, 1)))
    assert np.all(ids[:, 10:] == -1) and np.all(vals[:, 10:] == -np.inf)
    ids0, vals0 = run_topk_dev(np.zeros((3, 0), np.float32), 0, 5)
    assert np.all(ids0 == -1) and np.all(vals0 == -np.inf)


# ---------------------------------------------------------------------------
# the whole phase
# ---------------------------------------------------------------------------

def test_phase_with_fp32_queries_not_fp16_exact():
    """Conversion fixture: fp32 queries off the fp16 grid.  The oracle uses
    the unrounded fp32 values (the contract's first term covers operand
    rounding); the converted operand equals the oracle's conversion bit for
    bit, and the tail follows the fixed-order model on that operand."""
    base = qi.CONFIGS["nq256_nkv4096"]
    cfg = qi.Config("conv", 2, 96, base.H, base.D, 4096 + 21, 64, 16, "normal", 1012)
    w = qi.conversion_fixture(cfg)
    q32 = torch.from_numpy(w.q32).to(dev())
    kd = k_dev(w.kblk)
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                            keep_q16=True)
    ids = qsa.select_phase(q32, kd, cfg.n_kv, cfg.bs, cfg.k, ws)
    torch.cuda.synchronize()
    q16_gpu = ws.q16.cpu().numpy().view(np.uint16)
    assert np.array_equal(q16_gpu, oracle.convert_f32_f16(w.q32))
    s_gpu = ws.scores[:, :, :cfg.nb].reshape(cfg.rows, cfg.nb).cpu().numpy().astype(np.float64)
    ref = oracle.scores(w.q32, w.kblk, cfg.nb)
    check_bound(s_gpu, ref, "conversion")
    model = oracle.block_model_f32(q16_gpu, w.kblk, cfg.nf)
    assert np.array_equal(s_gpu[:, cfg.nf].astype(np.float32).view(np.uint32),
                          model.view(np.uint32))
    check_ids(ids.reshape(cfg.rows, cfg.k).cpu().numpy(), s_gpu, ref, cfg.k, "conversion")


# G, nq, H, D, n_kv, bs, k, tok_pad, q32 offset in floats.  16-byte aligned
# fp32 rows are read and converted by the scorers themselves (small rows, or
# no full block: the small scorer; G*ceil(nq/64) >= 256: the wide one); an
# offset of one float leaves the fp32 rows only 4-byte aligned, and the
# conversion kernel (strided for padded rows) runs first.
PHASE_CONV = [
    (2, 70, 12, 64, 65 * 64 + 5, 64, 8, 24, 0),    # padded rows, two head passes
    (2, 70, 12, 64, 65 * 64 + 5, 64, 8, 24, 1),    # padded rows, 4-byte aligned fp32
    (1, 33, 8, 128, 40, 64, 4, 8, 0),              # only a tail block
    (3, 129, 5, 128, 100 * 64 + 3, 64, 16, 0, 0),  # contiguous, odd H
    (1, 40, 8, 128, 10 * 64 + 7, 64, 8, 0, 1),     # contiguous, 4-byte aligned fp32
    (2, 5, 8, 128, 10 * 64 + 7, 64, 8, 24, 0),     # too few rows to stage: per-lane loads
    # wide rows: two block splits (only the first writes the workspace),
    # padded rows, two head passes
    (4, 4096, 12, 64, 40 * 64 + 5, 64, 8, 24, 0),
    (4, 4096, 3, 128, 70 * 64, 64, 8, 8, 0),       # wide, odd H, three tiles, no tail
    (4, 4096, 5, 128, 3 * 64 + 3, 64, 4, 0, 1),    # wide, 4-byte aligned: conversion kernel
    (4, 4096, 8, 128, 40, 64, 4, 0, 0),            # many rows, no full block: tail only
]


@pytest.mark.parametrize("case", PHASE_CONV,
                         ids=lambda c: "G{}_nq{}_H{}_D{}_nkv{}_bs{}_k{}_pad{}_off{}".format(*c))
def test_phase_conversion_paths(case):
    """The phase's conversion of fp32 queries gives the oracle's fp16 bits,
    writes exactly the token rows of the fp16 buffer (padding between rows
    untouched), and the scores, tail and ids follow from the fp32 inputs.
    Without the fp16 buffer the phase gives the same bits (16-byte aligned
    rows), or refuses cleanly (4-byte aligned rows)."""
    G, nq, H, D, n_kv, bs, k, tok_pad, off = case
    cfg = qi.Config("conv_path", G, nq, H, D, n_kv, bs, k, "normal", 4000 + nq)
    w = qi.conversion_fixture(cfg, seed=4000 + nq)
    row = G * H * D + tok_pad
    # fp32 rows at the requested offset from a 256-byte aligned allocation
    q32_buf = torch.full((off + nq * row,), float("nan"), dtype=torch.float32, device=dev())
    q32_rows = q32_buf[off:].view(nq, row)
    q32_rows[:, :G * H * D] = torch.from_numpy(w.q32.reshape(nq, -1)).to(dev())
    # fp16 workspace inside a canary-filled allocation (a signalling-NaN
    # pattern the conversion never produces: it quietens every NaN)
    sent16, pad16 = 0x7D5B, 4096
    q16_flat = torch.full((pad16 + nq * row + pad16,), sent16, dtype=torch.int16, device=dev())
    q16_view = q16_flat[pad16:pad16 + nq * row].view(nq, row)
    kd = k_dev(w.kblk)
    ld = -(-(cfg.nb + 1) // 32) * 32
    scores = torch.full((G, nq, ld), float("nan"), dtype=torch.float32, device=dev())
    ids = torch.full((G, nq, k), 123, dtype=torch.int32, device=dev())
    st = qsa.lib.qsa_select_phase(
        ctypes.c_void_p(q32_rows.data_ptr()), ctypes.c_void_p(q16_view.data_ptr()), row,
        ctypes.c_void_p(kd.data_ptr()), kd.stride(0), ctypes.c_void_p(scores.data_ptr()), ld,
        ctypes.c_void_p(ids.data_ptr()), k, None, G, nq, H, D, n_kv, bs, k, 0, 0, None)
    torch.cuda.synchronize()
    assert st == 0, qsa.status_string(st)
    flat = q16_flat.cpu().numpy()
    inside = flat[pad16:pad16 + nq * row].reshape(nq, row)
    assert np.all(flat[:pad16] == sent16) and np.all(flat[pad16 + nq * row:] == sent16)
    assert np.all(inside[:, G * H * D:] == sent16), "fp16 workspace written between token rows"
    got16 = inside[:, :G * H * D].view(np.uint16).reshape(nq, G, H, D)
    want16 = oracle.convert_f32_f16(w.q32)
    assert np.array_equal(got16, want16), "converted queries differ from the oracle's rounding"
    s_gpu = scores[:, :, :cfg.nb].reshape(cfg.rows, cfg.nb).cpu().numpy().astype(np.float64)
    ref = oracle.scores(w.q32, w.kblk, cfg.nb)
    check_bound(s_gpu, ref, "phase conversion")
    if cfg.nb > cfg.nf:
        model = oracle.block_model_f32(want16, w.kblk, cfg.nf)
        assert np.array_equal(s_gpu[:, cfg.nf].astype(np.float32).view(np.uint32),
                              model.view(np.uint32))
    check_ids(ids.reshape(cfg.rows, k).cpu().numpy(), s_gpu, ref, k, "phase conversion")

    scores2 = torch.full_like(scores, float("nan"))
    ids2 = torch.full_like(ids, 123)
    st = qsa.lib.qsa_select_phase(
        ctypes.c_void_p(q32_rows.data_ptr()), None, row,
        ctypes.c_void_p(kd.data_ptr()), kd.stride(0), ctypes.c_void_p(scores2.data_ptr()), ld,
        ctypes.c_void_p(ids2.data_ptr()), k, None, G, nq, H, D, n_kv, bs, k, 0, 0, None)
    torch.cuda.synchronize()
    if off % 4 != 0:
        assert st == qsa.QSA_ERR_UNSUPPORTED, qsa.status_string(st)
        assert torch.all(torch.isnan(scores2)) and torch.all(ids2 == 123)
    else:
        assert st == 0, qsa.status_string(st)
        nb = cfg.nb
        assert torch.equal(scores2[:, :, :nb].view(torch.int32), scores[:, :, :nb].view(torch.int32))
        assert torch.all(torch.isnan(scores2[:, :, nb:]))
        assert torch.equal(ids2, ids)


SPECIALS = np.array([0x7FC00001, 0xFFA00000, 0x7F800001, 0xFFFFFFFF,    # NaNs: payloads, signs, signalling
                     0x7F800000, 0xFF800000,                            # +-inf
                     0x47888000, 0xC77FF000, 0x477FE000, 0x477FEFFF,    # 70000 -> inf, -65520 -> -inf, 65504, just below the midpoint
                     0x358637BD, 0x33800000, 0x33000000, 0x33000001,    # 1e-6 (subnormal), 2^-24, 2^-25 (tie to 0), just above
                     0x80000000, 0x38800000], dtype=np.uint32)          # -0, 2^-14 (smallest normal)


@pytest.mark.parametrize("G,nq,off", [(1, 40, 0), (1, 40, 1), (4, 4096, 0)],
                         ids=["small_scorer", "conversion_kernel", "wide_scorer"])
def test_phase_converts_special_values(G, nq, off):
    """fp32 queries with NaNs (payloads, signs, signalling), infinities,
    overflow, the rounding at the fp16 maximum, subnormals and -0 in a few
    token rows.  With 16-byte aligned queries the scorer (small or wide)
    converts them on load; one float off, the conversion kernel does.  Either
    way the fp16 workspace holds the oracle's conversion bit for bit, and the
    rows without special values score within the bound."""
    H, D, n_kv, k = 8, 128, 5 * 64 + 3, 4
    cfg = qi.Config("specials", G, nq, H, D, n_kv, 64, k, "normal", 4321)
    w = qi.conversion_fixture(cfg, seed=4321)
    q32 = w.q32.copy()
    dirty = [3, 7, 30]
    for r in dirty:   # near the start of the token row and at its end (last KV head)
        flat = q32[r].reshape(-1).view(np.uint32)
        flat[5 * r:5 * r + len(SPECIALS)] = SPECIALS
        flat[flat.size - 5 * r - len(SPECIALS):flat.size - 5 * r] = SPECIALS
    buf = torch.zeros((off + q32.size,), dtype=torch.float32, device=dev())
    qd = buf[off:].view(nq, G, H, D)
    qd.copy_(torch.from_numpy(q32))
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                            keep_q16=True)
    ws.q16.view(torch.int16).fill_(0x7D5B)
    kd = k_dev(w.kblk)
    row = G * H * D
    st = qsa.lib.qsa_select_phase(
        ctypes.c_void_p(qd.data_ptr()), ctypes.c_void_p(ws.q16.data_ptr()), row,
        ctypes.c_void_p(kd.data_ptr()), kd.stride(0), ctypes.c_void_p(ws.scores.data_ptr()),
        ws.ld_s, ctypes.c_void_p(ws.ids.data_ptr()), k, None, G, nq, H, D, n_kv, 64, k, 0, 0,
        None)
    torch.cuda.synchronize()
    assert st == 0, qsa.status_string(st)
    got16 = ws.q16.cpu().numpy().view(np.uint16)
    want16 = oracle.convert_f32_f16(q32)
    assert np.array_equal(got16, want16), "converted queries differ from the oracle's rounding"
    clean = np.setdiff1d(np.arange(nq), dirty)
    s_gpu = ws.scores[:, clean, :cfg.nb].reshape(G * clean.size, cfg.nb).cpu().numpy()
    ref = oracle.scores(q32[clean], w.kblk, cfg.nb)
    check_bound(s_gpu.astype(np.float64), ref, "specials, clean rows")


@pytest.mark.parametrize("q_chunk", [0, 37, 64, 1000])
def test_phase_chunked_equals_whole(q_chunk):
    cfg = qi.Config("chunk", 3, 150, 8, 128, 70 * 64 + 5, 64, 32, "normal", 77)
    w = qi.make(cfg)
    q32 = torch.from_numpy(w.q32).to(dev())
    kd = k_dev(w.kblk)
    ws0 = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                             with_vals=True)
    ids0, vals0 = qsa.select_phase(q32, kd, cfg.n_kv, cfg.bs, cfg.k, ws0)
    wsc = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                             q_chunk=q_chunk, with_vals=True)
    idsc, valsc = qsa.select_phase(q32, kd, cfg.n_kv, cfg.bs, cfg.k, wsc)
    torch.cuda.synchronize()
    assert torch.equal(ids0, idsc) and torch.equal(vals0.view(torch.int32), valsc.view(torch.int32))
    s0 = ws0.scores[:, :, :cfg.nb].reshape(cfg.rows, cfg.nb).cpu().numpy().astype(np.float64)
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    check_bound(s0, ref, f"phase chunk={q_chunk}")
    check_ids(ids0.reshape(cfg.rows, cfg.k).cpu().numpy(), s0, ref, cfg.k, "phase")


def test_phase_ids_write_set():
    cfg = qi.TINY
    w = qi.make(cfg)
    ids = guarded((cfg.G, cfg.nq, cfg.k), torch.int32)
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev())
    ws.ids = ids.view
    qsa.select_phase(torch.from_numpy(w.q32).to(dev()), k_dev(w.kblk), cfg.n_kv, cfg.bs, cfg.k, ws)
    torch.cuda.synchronize()
    m = np.ones((cfg.G, cfg.nq, cfg.k), dtype=bool)
    assert ids.outside_intact(m) and ids.written_all(m)


def test_wide_and_small_scorers_agree_bitwise():
    """The whole query set takes the wide scorer (4096 rows per KV head),
    chunks of 1000 take the small one; both add the relu'd heads in the same
    order, so the chunked phase reproduces the whole phase bit for bit
    (scores of the last chunk, ids and values of every row)."""
    cfg = qi.Config("wn", 4, 4096, 8, 128, 30 * 64 + 11, 64, 16, "normal", 321)
    w = qi.make(cfg)
    q32 = torch.from_numpy(w.q32).to(dev())
    kd = k_dev(w.kblk)
    ws0 = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                             with_vals=True)
    ids0, vals0 = qsa.select_phase(q32, kd, cfg.n_kv, cfg.bs, cfg.k, ws0)
    wsc = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                             q_chunk=1000, with_vals=True)
    idsc, valsc = qsa.select_phase(q32, kd, cfg.n_kv, cfg.bs, cfg.k, wsc)
    torch.cuda.synchronize()
    assert torch.equal(ids0, idsc)
    assert torch.equal(vals0.view(torch.int32), valsc.view(torch.int32))
    # the chunked workspace holds the last chunk, queries 4000..4095, as
    # G x 96 consecutive rows
    n = cfg.nq - 4000
    last = wsc.scores.reshape(-1, wsc.ld_s)[:cfg.G * n].reshape(cfg.G, n, wsc.ld_s)[:, :, :cfg.nb]
    assert torch.equal(last.view(torch.int32), ws0.scores[:, 4000:, :cfg.nb].view(torch.int32))
    s0 = ws0.scores[:, :, :cfg.nb].reshape(cfg.rows, cfg.nb).cpu().numpy().astype(np.float64)
    model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
    assert np.array_equal(s0[:, cfg.nf].astype(np.float32).view(np.uint32), model.view(np.uint32))


# H, D: every row packing of the small scorer (head pairs 1, 2, 4, 8 per MFMA
# row block, padded heads for odd H), both head dims, one or two wide passes
SMALL_VS_WIDE = [(1, 128), (2, 64), (3, 128), (4, 64), (5, 128), (6, 128), (7, 64), (8, 128),
                 (8, 64), (12, 128), (16, 64)]


@pytest.mark.parametrize("H,D", SMALL_VS_WIDE, ids=lambda v: str(v))
def test_small_scorer_matches_wide_bitwise(H, D):
    """4 KV heads x 4096 queries take the wide scorer; a slice of 100 queries
    (few rows) takes the small scorer, which packs 16/NP queries x 2*NP heads
    into one MFMA row block instead of 16 queries x 2 heads.  The same MFMA
    dot products and the same head-sum order give the same bits, tail block
    included (no oracle needed: the two paths check each other)."""
    G, nq, t0, n = 4, 4096, 1234, 100
    cfg = qi.Config("small_vs_wide", G, nq, H, D, 20 * 64 + 9, 64, 4, "normal", 600 + 10 * H + D)
    w = qi.make(cfg)
    kd = k_dev(w.kblk)
    whole = qsa.block_scores(q_dev(w.q16), kd, cfg.n_kv, cfg.bs)
    part = qsa.block_scores(q_dev(w.q16[t0:t0 + n]), kd, cfg.n_kv, cfg.bs)
    torch.cuda.synchronize()
    assert torch.equal(part.contiguous().view(torch.int32),
                       whole[:, t0:t0 + n].contiguous().view(torch.int32))


# The wide scorer with several tiles per block split (4 KV heads x 4096
# queries: two splits of ceil(T/2) and floor(T/2) tiles): splits of one tile,
# shorter than the load distance; odd counts, the two-tile loop's remainder;
# both head dims; H = 12, whose second, accumulating head pass keeps the
# shorter load distance.
WIDE_TILES = [(64, 2, 8), (64, 5, 8), (64, 12, 8), (128, 3, 8), (128, 7, 8), (128, 5, 12)]


@pytest.mark.parametrize("D,n_tiles,H", WIDE_TILES, ids=lambda v: str(v))
def test_wide_scorer_tile_counts(D, n_tiles, H):
    """Wide-scorer bits equal the small scorer's on a slice of 100 queries,
    tail block included, and that slice is within the bound of the oracle."""
    G, nq, t0, n = 4, 4096, 777, 100
    cfg = qi.Config("wide_tiles", G, nq, H, D, n_tiles * 32 * 64 + 9, 64, 4, "normal",
                    1100 + 10 * n_tiles + D + H)
    log(f"wide scorer D={D} tiles={n_tiles} H={H}")
    w = qi.make(cfg)
    kd = k_dev(w.kblk)
    whole = qsa.block_scores(q_dev(w.q16), kd, cfg.n_kv, cfg.bs)
    part = qsa.block_scores(q_dev(w.q16[t0:t0 + n]), kd, cfg.n_kv, cfg.bs)
    torch.cuda.synchronize()
    sl = whole[:, t0:t0 + n].contiguous()
    assert torch.equal(part.contiguous().view(torch.int32), sl.view(torch.int32))
    s_gpu = sl.reshape(G * n, cfg.nb).cpu().numpy().astype(np.float64)
    check_bound(s_gpu, oracle.scores(w.q16[t0:t0 + n], w.kblk, cfg.nb), "wide tiles")


# More (KV head, query group) items than two workgroups per CU: the wide
# scorer's grid runs in more than one round of workgroups (520 to 1536 items,
# odd tile counts, one tile, partial query groups).
# (odd H and H = 6: heads zeroed or left out of the wide scorer's head quads,
# and the kept fp16 copy written for the real heads only)
MANY_ITEMS = [(8, 4100, 8, 128, 3), (16, 4096, 4, 64, 5), (17, 4000, 8, 128, 1),
              (12, 8192, 2, 128, 2), (8, 4096, 3, 128, 2), (4, 4100, 7, 64, 3),
              (4, 4096, 6, 128, 2), (8, 4096, 5, 64, 1), (4, 4096, 1, 128, 2)]


@pytest.mark.parametrize("H", [8, 5])
def test_wide_scorer_chunked_phase_keeps_q16(H):
    """A phase over 4 KV heads x 8300 queries in chunks of 4160: each chunk,
    the ragged second one (4140 queries) too, is 260 groups of 64 queries and
    takes the wide scorer, its fp32 queries converted on load and kept in the
    fp16 copy.  Ids, values and the kept copy are bit for bit those of one
    pass (and the copy the inputs' fp16 bits), the workspace holds the last
    chunk's scores, and every tail cell is the fixed-order model."""
    G, nq, D, bs, k, qc = 4, 8300, 128, 64, 64, 4160
    cfg = qi.Config("wide_chunked", G, nq, H, D, 40 * 64 + 11, bs, k, "normal", 1500 + H)
    log(f"wide scorer, chunked phase with the fp16 copy kept: H={H}")
    w = qi.make(cfg)
    q = torch.from_numpy(w.q32).to(dev())
    kb = k_dev(w.kblk)

    def run(chunk):
        ws = qsa.PhaseWorkspace(nq, G, H, D, cfg.n_kv, bs, k, dev(), with_vals=True,
                                q_chunk=chunk, keep_q16=True)
        ids, vals = qsa.select_phase(q, kb, cfg.n_kv, bs, k, ws)
        torch.cuda.synchronize()
        return ws, ids.cpu().numpy(), vals.cpu().numpy()

    ws1, ids1, v1 = run(0)
    wsc, idsc, vc = run(qc)
    nb = cfg.nb
    assert wsc.chunk_rows == qc
    assert np.array_equal(idsc, ids1)
    assert np.array_equal(vc.view(np.uint32), v1.view(np.uint32))
    assert np.array_equal(ws1.q16.cpu().numpy().view(np.uint16), w.q16)
    assert np.array_equal(wsc.q16.cpu().numpy().view(np.uint16), w.q16)
    n = nq - qc
    last = wsc.scores.reshape(-1, wsc.ld_s)[:G * n].reshape(G, n, wsc.ld_s)[:, :, :nb]
    assert torch.equal(last.view(torch.int32), ws1.scores[:, qc:, :nb].view(torch.int32))
    s_all = ws1.scores[:, :, :nb].reshape(cfg.rows, nb)
    model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
    assert np.array_equal(s_all[:, cfg.nf].cpu().numpy().view(np.uint32), model.view(np.uint32))


@pytest.mark.parametrize("G,nq,H,D,n_tiles", MANY_ITEMS, ids=lambda v: str(v))
def test_wide_scorer_many_items(G, nq, H, D, n_tiles):
    """The wide scorer over more work items than one round of workgroups:
    the fp16-input scores and the phase's fp32-input scores are the same
    bits, a slice of queries scored by the small scorer too, every tail cell
    is the fixed-order model, the kept fp16 copy is exactly the oracle's
    conversion, and the rows of every query group edge are within the bound
    of the oracle."""
    cfg = qi.Config("many_items", G, nq, H, D, n_tiles * 32 * 64 + 7, 64, 8, "normal",
                    1300 + G + n_tiles + H)
    log(f"wide scorer, many items: G={G} nq={nq} H={H} D={D} tiles={n_tiles}")
    w = qi.make(cfg)
    kd = k_dev(w.kblk)
    nb = cfg.nb
    whole = qsa.block_scores(q_dev(w.q16), kd, cfg.n_kv, cfg.bs)
    t0, n = 1000, 70
    part = qsa.block_scores(q_dev(w.q16[t0:t0 + n]), kd, cfg.n_kv, cfg.bs)
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                            keep_q16=True)
    ids = qsa.select_phase(torch.from_numpy(w.q32).to(dev()), kd, cfg.n_kv, cfg.bs, cfg.k, ws)
    torch.cuda.synchronize()
    assert torch.equal(part.contiguous().view(torch.int32),
                       whole[:, t0:t0 + n].contiguous().view(torch.int32))
    assert torch.equal(ws.scores[:, :, :nb].contiguous().view(torch.int32),
                       whole.contiguous().view(torch.int32))
    assert np.array_equal(ws.q16.cpu().numpy().view(np.uint16), w.q16)
    s_all = whole.reshape(cfg.rows, nb)
    model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
    assert np.array_equal(s_all[:, cfg.nf].cpu().numpy().view(np.uint32), model.view(np.uint32))
    edges = sorted({g * nq + t for g in range(G) for t in (0, 63, 64, 1023, 1024, nq - 65,
                                                          nq - 64, nq - 1)})
    rows = np.array(edges, dtype=np.int64)
    s_gpu = s_all[torch.from_numpy(rows).to(dev())].cpu().numpy().astype(np.float64)
    ref = oracle.scores(w.q16, w.kblk, nb, rows=rows)
    check_bound(s_gpu, ref, "many items")
    got = ids.reshape(cfg.rows, cfg.k)[torch.from_numpy(rows).to(dev())].cpu().numpy()
    check_ids(got, s_gpu, ref, cfg.k, "many items")


# 256 queries of one KV head at H = 8 give 16 groups of four query groups,
# so the block axis is cut into 16 segments of n_tiles/16 tiles: 2, 3, 4 and
# 6 tiles per segment, eight waves (two per query group, each taking half of
# every staged chunk), K staged one tile per wave half and barrier (2, 3, 6)
# or two (4).
SMALL_CHUNKS = [32, 48, 64, 96]


@pytest.mark.parametrize("n_tiles", SMALL_CHUNKS, ids=lambda v: f"tiles{v}")
def test_small_scorer_chunking(n_tiles):
    """The small scorer over 2-6 tiles per block segment, both K staging
    depths, with a tail block: the phase on fp32 queries gives scores within
    the bound, the tail bit for bit the fixed-order model, ids exact on the
    device scores, and the same bits as the fp16-input entry point."""
    cfg = qi.Config("chunks", 1, 256, 8, 128, n_tiles * 32 * 64 + 13, 64, 16, "normal",
                    900 + n_tiles)
    log(f"small scorer, {n_tiles} tiles")
    w = qi.make(cfg)
    kd = k_dev(w.kblk)
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev())
    ids = qsa.select_phase(torch.from_numpy(w.q32).to(dev()), kd, cfg.n_kv, cfg.bs, cfg.k, ws)
    s16 = qsa.block_scores(q_dev(w.q16), kd, cfg.n_kv, cfg.bs)
    torch.cuda.synchronize()
    nb = cfg.nb
    assert torch.equal(ws.scores[:, :, :nb].contiguous().view(torch.int32),
                       s16.contiguous().view(torch.int32))
    s_gpu = ws.scores[:, :, :nb].reshape(cfg.rows, nb).cpu().numpy().astype(np.float64)
    ref = oracle.scores(w.q16, w.kblk, nb)
    check_bound(s_gpu, ref, "small chunks")
    model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
    assert np.array_equal(s_gpu[:, cfg.nf].astype(np.float32).view(np.uint32), model.view(np.uint32))
    check_ids(ids.reshape(cfg.rows, cfg.k).cpu().numpy(), s_gpu, ref, cfg.k, "small chunks")


# Slices of 100 queries (4 KV heads) that the small scorer serves with eight
# waves (segments of two or more tiles): every head packing (H = 2, 4, 5, 8,
# 12, 16), both head dims, 4-tile chunks (40 and 64 tiles) and 2-tile chunks
# over a ragged last segment (24 tiles: segments of 3), with and without the
# partial block.
EIGHT_WAVES = [(8, 128, 40, True), (8, 128, 24, False), (2, 64, 40, True), (4, 128, 64, True),
               (16, 128, 40, False), (12, 64, 24, True), (5, 128, 40, True), (8, 64, 16, True)]


@pytest.mark.parametrize("H,D,n_tiles,tail", EIGHT_WAVES, ids=lambda v: str(v))
def test_small_scorer_eight_waves_bitwise(H, D, n_tiles, tail):
    """The eight-wave small scorer gives the wide scorer's bits: on fp16
    queries (staged through LDS) and in the phase on fp32 queries (converted
    on load, the kept fp16 copy exactly the input's bits), tail included."""
    G, nq, t0, n = 4, 4096, 1500, 100
    n_kv = n_tiles * 32 * 64 + (9 if tail else 0)
    cfg = qi.Config("eight_waves", G, nq, H, D, n_kv, 64, 8, "normal", 1400 + 10 * H + n_tiles + D)
    log(f"small scorer, eight waves: H={H} D={D} tiles={n_tiles} tail={tail}")
    w = qi.make(cfg)
    kd = k_dev(w.kblk)
    nb = cfg.nb
    whole = qsa.block_scores(q_dev(w.q16), kd, n_kv, cfg.bs)
    part = qsa.block_scores(q_dev(w.q16[t0:t0 + n]), kd, n_kv, cfg.bs)
    ws = qsa.PhaseWorkspace(n, G, H, D, n_kv, cfg.bs, cfg.k, dev(), keep_q16=True)
    q32 = torch.from_numpy(np.ascontiguousarray(w.q32[t0:t0 + n])).to(dev())
    qsa.select_phase(q32, kd, n_kv, cfg.bs, cfg.k, ws)
    torch.cuda.synchronize()
    ref = whole[:, t0:t0 + n].contiguous().view(torch.int32)
    assert torch.equal(part.contiguous().view(torch.int32), ref)
    assert torch.equal(ws.scores[:, :, :nb].contiguous().view(torch.int32), ref)
    assert np.array_equal(ws.q16.cpu().numpy().view(np.uint16), w.q16[t0:t0 + n])


def test_wide_scorer_global_store_path():
    """The wide scorer's plain global-store path (a KV head's score region of
    2^30 bytes or more), with two head passes and the tail in the same
    launches: write set and bound."""
    cfg = qi.Config("wide_g", 4, 4096, 12, 128, 9 * 64 + 5, 64, 8, "normal", 98)
    w = qi.make(cfg)
    ld = 1 << 16                                   # 4096 rows x 256 KiB: 1 GiB per KV head
    sent = int(SENTINEL)
    out = torch.full((cfg.G, cfg.nq, ld), sent, dtype=torch.int32, device=dev())
    qsa.block_scores(q_dev(w.q16), k_dev(w.kblk), cfg.n_kv, cfg.bs, out=out.view(torch.float32))
    torch.cuda.synchronize()
    head = out[:, :, :cfg.nb + 256]
    assert torch.all(head[:, :, cfg.nb:] == sent), "write past nb"
    assert torch.all(out[:, :, ld - 256:] == sent)
    assert not torch.any(head[:, :, :cfg.nb] == sent), "cell not written"
    s_gpu = head[:, :, :cfg.nb].view(torch.float32).reshape(cfg.rows, cfg.nb).cpu().numpy()
    del out, head
    torch.cuda.empty_cache()
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    check_bound(s_gpu.astype(np.float64), ref, "wide scorer, global stores")
    model = oracle.block_model_f32(w.q16, w.kblk, cfg.nf)
    assert np.array_equal(s_gpu[:, cfg.nf].view(np.uint32), model.view(np.uint32))


def test_wide_rows_use_global_store_path():
    """A score region past 2^30 bytes per KV head takes the scorer's plain
    global-store path (the buffer-store path needs 30-bit offsets); it must
    give the same write set and the same bound.  Few query rows: the small
    scorer, whose 64-bit addressing covers the region, with H = 12 in one
    row block of two queries x 16 head slots."""
    cfg = qi.Config("wide", 1, 70, 12, 128, 65 * 64 + 5, 64, 8, "normal", 99)
    w = qi.make(cfg)
    ld = 1 << 24                                   # 64 MiB per row: 4.4 GiB region
    sent = int(SENTINEL)
    out = torch.full((cfg.G, cfg.nq, ld), sent, dtype=torch.int32, device=dev())
    qsa.block_scores(q_dev(w.q16), k_dev(w.kblk), cfg.n_kv, cfg.bs, out=out.view(torch.float32))
    torch.cuda.synchronize()
    head = out[:, :, :cfg.nb + 256]
    assert torch.all(head[:, :, cfg.nb:] == sent), "write past nb"
    assert torch.all(out[:, :, ld - 256:] == sent)
    assert not torch.any(head[:, :, :cfg.nb] == sent), "cell not written"
    s_gpu = head[:, :, :cfg.nb].view(torch.float32).reshape(cfg.rows, cfg.nb).cpu().numpy()
    ref = oracle.scores(w.q16, w.kblk, cfg.nb)
    check_bound(s_gpu.astype(np.float64), ref, "wide rows")
    del out
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# the forced-tail rule (QSA_FORCE_TAIL): 1e9 added to the partial block's
# score after its head sum, on every path that scores that block
# ---------------------------------------------------------------------------

FORCED = [
    # G, nq, H, D, n_kv, bs: path
    (1, 37, 4, 64, 1000, 64),          # small scorer, tail segment
    (8, 1, 8, 128, 131109, 64),        # the decode step: small scorer, one query per KV head
    (4, 4096, 8, 128, 40 * 64 + 5, 64),    # wide scorer, tail in the same launch
    (2, 8192, 12, 64, 20 * 64 + 9, 64),    # wide scorer, two head passes (the rule on the last)
    (4, 4200, 8, 128, 40, 64),         # only a tail block: the standalone tail kernel
    (1, 50, 16, 128, 18 * 64, 64),     # no partial block: the flag changes nothing
]


@pytest.mark.parametrize("geo", FORCED, ids=lambda g: "G{}_nq{}_H{}_D{}_nkv{}".format(*g[:5]))
def test_force_tail_scores_and_selection(geo):
    G, nq, H, D, n_kv, bs = geo
    k = 16
    cfg = qi.Config("forced", G, nq, H, D, n_kv, bs, k, "normal", 900 + nq)
    w = qi.make(cfg)
    log(f"forced tail {geo}")
    qd, kd = q_dev(w.q16), k_dev(w.kblk)
    s0 = qsa.block_scores(qd, kd, n_kv, bs).cpu().numpy().reshape(G * nq, cfg.nb)
    s1 = qsa.block_scores(qd, kd, n_kv, bs, force_tail=True).cpu().numpy().reshape(G * nq, cfg.nb)
    torch.cuda.synchronize()
    nf = cfg.nf
    # the full blocks are untouched by the flag, bit for bit
    assert np.array_equal(s0[:, :nf].view(np.uint32), s1[:, :nf].view(np.uint32))
    if cfg.nb == nf:
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))
        return
    # the tail bit for bit the fixed-order model with the rule, and within the
    # rule's bound of the exact forced score
    model = oracle.block_model_f32(w.q16, w.kblk, nf, force_tail=True)
    assert np.array_equal(s1[:, nf].view(np.uint32), model.view(np.uint32))
    rows = np.arange(min(G * nq, 512), dtype=np.int64) * max(1, (G * nq) // 512)
    rows = np.unique(np.minimum(rows, G * nq - 1))
    ref = oracle.force_tail(oracle.scores(w.q16, w.kblk, cfg.nb, rows=rows), n_kv, bs)
    check_bound(s1[rows].astype(np.float64), ref, "forced")
    # the phase with the rule selects the tail first in every row
    ws = qsa.PhaseWorkspace(nq, G, H, D, n_kv, bs, k, dev())
    ids = qsa.select_phase(torch.from_numpy(w.q32).to(dev()), kd, n_kv, bs, k, ws,
                           force_tail=True).cpu().numpy().reshape(G * nq, k)
    sc = ws.scores[:, :, :cfg.nb].cpu().numpy().reshape(G * nq, cfg.nb)
    assert np.array_equal(sc.view(np.uint32), s1.view(np.uint32))
    assert np.all(ids[:, 0] == nf)
    check_ids(ids[rows], sc[rows].astype(np.float64), ref, k, "forced phase")


# ---------------------------------------------------------------------------
# the decode scorer (one MFMA row block of queries per KV head) against the
# small scorer: a query's scores depend on that query alone, so the decode
# rows must equal the same queries' rows scored among many (small scorer),
# bit for bit, and the oracle's bound
# ---------------------------------------------------------------------------

DECODE_VS_SMALL = [
    # G, nq (decode), H, D, n_kv
    (8, 1, 8, 128, 131109),     # the decode step
    (8, 4, 8, 128, 4096 + 3),   # a full row block of 4 queries x 8 heads
    (2, 8, 4, 64, 33 * 64),     # 8 queries x 4 heads, no tail
    (3, 2, 12, 128, 95 * 64 + 1),   # 2 queries x 16 head slots (H = 12)
    (1, 16, 1, 64, 40 * 64 + 7),    # 16 queries x one head
    (4, 3, 5, 128, 31),         # no full block: the small scorer's tail-only path
]


@pytest.mark.parametrize("geo", DECODE_VS_SMALL, ids=lambda g: "G{}_nq{}_H{}_D{}_nkv{}".format(*g))
def test_decode_scorer_matches_small_bitwise(geo):
    G, nq, H, D, n_kv = geo
    big = 80   # 80 queries per KV head: the small scorer
    cfg = qi.Config("dec", G, big, H, D, n_kv, 64, 8, "normal", 7700 + nq + H)
    w = qi.make(cfg)
    log(f"decode vs small {geo}")
    q_all = torch.from_numpy(w.q32).to(dev())
    kd = k_dev(w.kblk)
    ws_big = qsa.PhaseWorkspace(big, G, H, D, n_kv, 64, 8, dev())
    qsa.select_phase(q_all, kd, n_kv, 64, 8, ws_big)
    ws_dec = qsa.PhaseWorkspace(nq, G, H, D, n_kv, 64, 8, dev(), keep_q16=True)
    qsa.select_phase(q_all[:nq].contiguous(), kd, n_kv, 64, 8, ws_dec)
    torch.cuda.synchronize()
    nb = cfg.nb
    a = ws_big.scores[:, :nq, :nb].cpu().numpy()
    b = ws_dec.scores[:, :, :nb].cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "decode rows differ from the small scorer's"
    assert np.array_equal(ws_big.ids[:, :nq].cpu().numpy(), ws_dec.ids.cpu().numpy())
    # the fp16 queries the decode scorer wrote are the conversion's
    assert np.array_equal(ws_dec.q16.cpu().numpy().view(np.uint16), w.q16[:nq])
    ref = oracle.scores(w.q16[:nq], w.kblk, nb)
    check_bound(b.reshape(G * nq, nb).astype(np.float64), ref, "decode")
