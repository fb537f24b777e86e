"""GPU parity of the streaming selection (QSA_STREAM_SELECT): the wide scorer
keeps a running candidate set per score row while the block tiles stream by
and writes no score.  Its ids and values must be bit for bit those of the
phase with the separate selector launch (which the other parity tests hold to
the oracle), and the score workspace must be left untouched, on every shape
it serves (one workgroup per 64 queries over all blocks, H <= 8, nb <= 65536)
and through the phase's options (fp16 or fp32 queries, a kept fp16 copy,
query chunks, values, the forced-tail rule, the allocation-free entry point).

The inputs cover the paths of the running selection: random scores (a few
compactions per row, the 16-bit threshold), rows that never fill their
buffer (nb <= 128), scores that rise with the block id (every block admitted,
a compaction every tile or two), scores that fall (nothing admitted after
the first tiles), integer scores with many ties and all-equal rows (the exact
cut of ties in id order), and non-finite scores (NaN admitted, ranked last).
Sampled rows of the prefill chunk are also checked against the oracle's
top-k of the oracle scores within its near-tie rule."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
from gpu_util import dev, log

pytestmark = pytest.mark.gpu

import sparse_attention_block_qsa_amd as qsa  # noqa: E402

CANARY = 0x7FC0BEEF   # a NaN pattern no scorer writes


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _phase(w, cfg, stream, q_chunk=0, fp16=False, force_tail=False, keep_q16=False):
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                            q_chunk=q_chunk, with_vals=True, keep_q16=keep_q16)
    q = (torch.from_numpy(w.q16.view(np.float16)).to(dev()) if fp16
         else torch.from_numpy(w.q32).to(dev()))
    kd = torch.from_numpy(w.kblk.view(np.float16)).to(dev())
    ws.ids.fill_(-7)
    ws.vals.fill_(float("nan"))
    ws.scores.view(torch.int32).fill_(CANARY)
    if ws.q16 is not None:
        ws.q16.view(torch.int16).fill_(-1)
    qsa.select_phase(q, kd, cfg.n_kv, cfg.bs, cfg.k, ws, force_tail=force_tail,
                     stream_select=stream)
    torch.cuda.synchronize()
    return ws


def _same(a, b, name):
    assert torch.equal(a.ids, b.ids), f"{name}: ids differ"
    assert torch.equal(a.vals.view(torch.int32), b.vals.view(torch.int32)), f"{name}: vals differ"
    assert int((b.ids == -7).sum()) == 0, f"{name}: ids not written"


def _untouched(ws, name):
    assert bool((ws.scores.view(torch.int32) == CANARY).all()), f"{name}: score workspace written"


def _workload(cfg, q, k):
    """A workload from float64 query [nq][G][H][D] and key [G][nb][D] values."""
    q16 = qi.f64_to_f16_bits(q)
    return qi.Workload(cfg, q16, qi.f64_to_f16_bits(k), qi.f16_bits_to_f32(q16))


# (name, G, nq, H, D, n_kv, k, q_chunk, fp16 queries, forced tail)
CASES = [
    ("prefill", 4, 16384, 8, 128, 131077, 64, 0, False, False),
    ("prefill_chunked", 4, 16384, 8, 128, 131077, 64, 8192, False, False),
    ("prefill_fp16_forced", 4, 16384, 8, 128, 131077, 64, 0, True, True),
    ("nb101_fills_never", 8, 4096, 8, 128, 100 * 64 + 7, 64, 0, False, False),
    ("nb128_exact", 8, 4096, 8, 128, 128 * 64, 64, 0, False, False),
    ("nb129_tail", 8, 4096, 8, 128, 128 * 64 + 1, 64, 0, False, False),
    ("nb701_k32", 8, 4096, 8, 128, 700 * 64 + 5, 32, 0, False, False),
    ("nb1024_d64_h5_k16", 8, 4100, 5, 64, 1024 * 64, 16, 0, False, False),
    ("nb2112_h3_k7", 16, 2048, 3, 64, 2112 * 64, 7, 0, True, False),
    ("nb4099_h1_k1", 8, 4096, 1, 128, 4098 * 64 + 33, 1, 0, False, False),
    ("nb8193_h8_k64", 4, 8192, 8, 128, 8193 * 64, 64, 0, False, True),
    ("nb300_h7_ragged_nq", 7, 5003, 7, 128, 299 * 64 + 63, 48, 0, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_stream_select_equals_separate_selector(case):
    name, G, nq, H, D, n_kv, k, q_chunk, fp16, forced = case
    cfg = qi.Config(name, G, nq, H, D, n_kv, 64, k, "normal", 5000 + G + H + k)
    w = qi.make(cfg)
    log(f"stream select {case}")
    a = _phase(w, cfg, False, q_chunk, fp16, forced)
    b = _phase(w, cfg, True, q_chunk, fp16, forced)
    _same(a, b, name)
    _untouched(b, name)
    if name == "prefill":
        # sampled rows against the oracle: the device selection is the
        # oracle's, up to near-ties of the oracle scores
        nb = cfg.nb
        rows = np.unique(np.linspace(0, G * nq - 1, 64).astype(np.int64))
        ids = b.ids.reshape(G * nq, k)[torch.from_numpy(rows).to(dev())].cpu().numpy()
        ref = oracle.scores(w.q16, w.kblk, nb, rows=rows)
        sel = oracle.check_selection(ids, ref, k)
        log(f"  [{name}] rows differing {sel.rows_differing}, worst gap/2B {sel.worst_gap_ratio:.3f}")
        assert sel.ok, sel.detail


def test_stream_select_keeps_fp16_copy():
    """With an fp16 buffer kept, the streaming scorer stores the same
    conversion as the two-launch phase."""
    cfg = qi.Config("keep16", 8, 4096, 8, 128, 600 * 64 + 9, 64, 64, "normal", 5101)
    w = qi.make(cfg)
    a = _phase(w, cfg, False, keep_q16=True)
    b = _phase(w, cfg, True, keep_q16=True)
    _same(a, b, "keep16")
    _untouched(b, "keep16")
    assert torch.equal(a.q16.view(torch.int16), b.q16.view(torch.int16))


def _ramp_case(name, sign, nb=1500, G=4, nq=8192, H=8, D=128, k=64, tail=17):
    """Positive queries and keys whose scale rises (sign > 0) or falls with
    the block id: every row's scores are monotone in the block id."""
    n_kv = nb * 64 + tail
    cfg = qi.Config(name, G, nq, H, D, n_kv, 64, k, "normal", 0)
    nbt = cfg.nb
    rng = np.random.default_rng(11)
    q = np.abs(rng.standard_normal((nq, G, H, D))) / math.sqrt(D)
    base = np.abs(rng.standard_normal((G, 1, D))) / math.sqrt(D)
    ramp = np.linspace(0.25, 4.0, nbt)[None, :, None]
    if sign < 0:
        ramp = ramp[:, ::-1, :]
    return cfg, _workload(cfg, q, base * ramp)


@pytest.mark.parametrize("sign", [1, -1], ids=["rising", "falling"])
def test_stream_select_monotone_scores(sign):
    """Rising scores admit every block (a compaction every tile or two);
    falling ones admit nothing after the first tiles."""
    cfg, w = _ramp_case(f"ramp{sign}", sign)
    a = _phase(w, cfg, False)
    b = _phase(w, cfg, True)
    _same(a, b, cfg.name)
    _untouched(b, cfg.name)


@pytest.mark.parametrize("kind", ["integer", "coded", "binary", "all_zero", "all_equal"])
def test_stream_select_ties(kind):
    """Many equal scores: the compactions take the exact cut (ties in id
    order), and rows where every score is equal keep the first k ids."""
    G, nq, H, D, k = 8, 4096, 8, 128, 64
    n_kv = 1100 * 64 + 40
    cfg = qi.Config(f"ties_{kind}", G, nq, H, D, n_kv, 64, k, "normal", 5200)
    nb = cfg.nb
    if kind == "integer":
        w = qi.integer_fixture(cfg)
    elif kind == "coded":
        w = qi.coded_fixture(cfg)
    else:
        rng = np.random.default_rng(13)
        if kind == "binary":
            q = (rng.random((nq, G, H, D)) < 0.05).astype(np.float64)
            kk = (rng.random((G, nb, D)) < 0.05).astype(np.float64)
        elif kind == "all_zero":
            q = rng.standard_normal((nq, G, H, D))
            kk = np.zeros((G, nb, D))
        else:
            # small integers times 0.5: every block's score is exact in any
            # order, so the tail block's fixed-order score equals the others
            q = rng.integers(1, 4, size=(nq, G, H, D)).astype(np.float64)
            kk = np.ones((G, nb, D)) * 0.5
        w = _workload(cfg, q, kk)
    a = _phase(w, cfg, False)
    b = _phase(w, cfg, True)
    _same(a, b, cfg.name)
    _untouched(b, cfg.name)
    if kind in ("all_zero", "all_equal"):
        want = torch.arange(k, dtype=torch.int32, device=dev()).expand(G, nq, k)
        assert torch.equal(b.ids, want)


def test_stream_select_non_finite_scores():
    """Infinite queries give NaN and infinite scores (outside the inputs'
    contract, but the selection of those scores must still match): NaN is
    admitted and ranked below every number."""
    G, nq, H, D, k = 8, 4096, 8, 128, 64
    cfg = qi.Config("nonfinite", G, nq, H, D, 700 * 64 + 3, 64, k, "normal", 5301)
    w = qi.make(cfg)
    q16 = w.q16.copy()
    q16[::3, :, 0, 5] = 0x7C00            # +inf in one channel of every third query
    q16[1::7, :, 2, :] = 0x7C00           # whole heads at +inf
    w = qi.Workload(cfg, q16, w.kblk, qi.f16_bits_to_f32(q16))
    a = _phase(w, cfg, False, fp16=True)
    b = _phase(w, cfg, True, fp16=True)
    assert torch.isnan(a.vals).any() or torch.isinf(a.vals).any()
    _same(a, b, cfg.name)
    _untouched(b, cfg.name)


def test_stream_select_noalloc_equals_phase():
    """The allocation-free entry point with the streaming selection: one pass
    without the scratch array.  A q_chunk of all the queries, which the array
    cannot hold (about 2016 queries fit at this shape), is refused without
    the flag and served with it, so the streaming path is the one taken."""
    cfg = qi.Config("noalloc_stream", 4, 8192, 8, 128, 2049 * 64 - 20, 64, 64, "normal", 5401)
    w = qi.make(cfg)
    a = _phase(w, cfg, False)
    q = torch.from_numpy(w.q32).to(dev())
    kd = torch.from_numpy(w.kblk.view(np.float16)).to(dev())
    ids = torch.full((cfg.G, cfg.nq, cfg.k), -7, dtype=torch.int32, device=dev())
    vals = torch.full((cfg.G, cfg.nq, cfg.k), float("nan"), device=dev())
    with pytest.raises(qsa.QSAError) as err:
        qsa.select_phase_noalloc(q, kd, cfg.n_kv, cfg.bs, cfg.k, ids, vals, q_chunk=cfg.nq)
    assert err.value.status == qsa.QSA_ERR_TOO_LARGE
    for q_chunk in (0, cfg.nq):
        ids.fill_(-7)
        vals.fill_(float("nan"))
        qsa.select_phase_noalloc(q, kd, cfg.n_kv, cfg.bs, cfg.k, ids, vals, q_chunk=q_chunk,
                                 stream_select=True)
        torch.cuda.synchronize()
        assert torch.equal(a.ids, ids)
        assert torch.equal(a.vals.view(torch.int32), vals.view(torch.int32))


def test_stream_flag_on_shapes_it_does_not_serve():
    """Shapes outside the streaming form (few rows, more than 8 heads) take
    the two-launch path with the flag set, with the same results."""
    for cfg in (qi.HEADLINE, qi.DECODE,
                qi.Config("h12", 4, 8192, 12, 64, 300 * 64, 64, 32, "normal", 5501)):
        w = qi.make(cfg)
        a = _phase(w, cfg, False)
        b = _phase(w, cfg, True)
        _same(a, b, cfg.name)
        nb = cfg.nb
        assert torch.equal(a.scores[:, :, :nb].view(torch.int32),
                           b.scores[:, :, :nb].view(torch.int32))


def test_stream_select_random_geometries():
    """Seeded random shapes the streaming form serves (and a few it does not):
    ids and values equal the two-launch phase's, bit for bit."""
    rng = np.random.default_rng(20261202)
    for i in range(10):
        H = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8]))
        D = int(rng.choice([64, 128]))
        G = int(rng.choice([4, 8]))
        nq = int(rng.integers(4096, 4500) if G == 8 else rng.integers(8192, 8600))
        nb = int(rng.integers(40, 2500))
        n_kv = nb * 64 - int(rng.integers(0, 64))
        k = int(rng.integers(1, 65))
        cfg = qi.Config(f"rand{i}", G, nq, H, D, n_kv, 64, k, "normal", 6000 + i)
        w = qi.make(cfg)
        log(f"random stream geometry {i}: G {G} nq {nq} H {H} D {D} n_kv {n_kv} k {k}")
        a = _phase(w, cfg, False, fp16=bool(i % 2))
        b = _phase(w, cfg, True, fp16=bool(i % 2))
        _same(a, b, cfg.name)
