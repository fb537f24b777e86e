"""GPU parity of the fused selection (QSA_FUSED_SELECT): the wide scorer
selects each row's top-k inside its own launch.  Its ids, values and scores
must be bit for bit those of the phase with the separate selector launch
(which the other parity tests hold to the oracle), on every shape the fused
form serves (513-1024 or 2049-2112 blocks, one workgroup per query group, H
<= 8) and through the phase's options: fp16 or fp32 queries, query chunks,
values, the forced-tail rule.  Sampled rows are also checked against the
oracle's top-k of the device scores and its near-tie rule."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
from gpu_util import dev, log

pytestmark = pytest.mark.gpu

import sparse_attention_block_qsa_amd as qsa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _phase(w, cfg, fused, q_chunk=0, fp16=False, force_tail=False):
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                            q_chunk=q_chunk, with_vals=True)
    q = (torch.from_numpy(w.q16.view(np.float16)).to(dev()) if fp16
         else torch.from_numpy(w.q32).to(dev()))
    kd = torch.from_numpy(w.kblk.view(np.float16)).to(dev())
    ws.ids.fill_(-7)
    ws.vals.fill_(float("nan"))
    qsa.select_phase(q, kd, cfg.n_kv, cfg.bs, cfg.k, ws, force_tail=force_tail,
                     fused_select=fused)
    torch.cuda.synchronize()
    return ws


# (name, G, nq, H, D, n_kv, k, q_chunk, fp16 queries, forced tail)
CASES = [
    ("prefill", 4, 16384, 8, 128, 131077, 64, 0, False, False),
    ("prefill_chunked", 4, 16384, 8, 128, 131077, 64, 8192, False, False),
    ("prefill_fp16_forced", 4, 16384, 8, 128, 131077, 64, 0, True, True),
    ("nb701_k32", 8, 4096, 8, 128, 700 * 64 + 5, 32, 0, False, False),
    ("nb1024_d64_h5", 8, 4100, 5, 64, 1024 * 64, 16, 0, False, False),
    ("nb2112_h3_k7", 16, 2048, 3, 64, 2112 * 64, 7, 0, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_fused_select_equals_separate_selector(case):
    name, G, nq, H, D, n_kv, k, q_chunk, fp16, forced = case
    cfg = qi.Config(name, G, nq, H, D, n_kv, 64, k, "normal", 4000 + G + H)
    w = qi.make(cfg)
    log(f"fused select {case}")
    a = _phase(w, cfg, False, q_chunk, fp16, forced)
    b = _phase(w, cfg, True, q_chunk, fp16, forced)
    assert torch.equal(a.ids, b.ids), f"{name}: ids differ"
    assert torch.equal(a.vals.view(torch.int32), b.vals.view(torch.int32)), f"{name}: vals differ"
    nb = cfg.nb
    assert torch.equal(a.scores[:, :, :nb].view(torch.int32), b.scores[:, :, :nb].view(torch.int32))
    assert int((b.ids == -7).sum()) == 0
    if q_chunk == 0:
        # sampled rows against the oracle: ids exactly the top-k of the device
        # scores, and the oracle's selection up to near-ties
        rows = np.unique(np.linspace(0, G * nq - 1, 96).astype(np.int64))
        s_dev = b.scores[:, :, :nb].reshape(G * nq, nb)[torch.from_numpy(rows).to(dev())]
        s_dev = s_dev.cpu().numpy().astype(np.float64)
        ids = b.ids.reshape(G * nq, k)[torch.from_numpy(rows).to(dev())].cpu().numpy()
        assert np.array_equal(ids, oracle.topk(s_dev, k)[0])
        ref = oracle.scores(w.q16, w.kblk, nb, rows=rows)
        if forced:
            ref = oracle.force_tail(ref, n_kv, 64)
        sel = oracle.check_selection(ids, ref, k)
        log(f"  [{name}] rows differing {sel.rows_differing}, worst gap/2B {sel.worst_gap_ratio:.3f}")
        assert sel.ok, sel.detail


def test_fused_flag_on_shapes_it_does_not_serve():
    """Shapes outside the fused form (few rows, other block counts) take the
    separate selector with the flag set, with the same results."""
    for cfg in (qi.HEADLINE, qi.DECODE, qi.Config("x", 4, 8192, 8, 128, 40 * 64, 64, 16, "normal", 7)):
        w = qi.make(cfg)
        a = _phase(w, cfg, False)
        b = _phase(w, cfg, True)
        assert torch.equal(a.ids, b.ids) and torch.equal(a.vals.view(torch.int32),
                                                         b.vals.view(torch.int32))
