"""qsa_select_phase_noalloc, the phase for callers that cannot allocate,
through the C ABI: the same ids and values, bit for bit, as qsa_select_phase
with the same query chunking, on two calls in a row whose second input is
smaller; a shape whose scores exceed the fixed scratch array is walked in
chunks and still gives the one-pass result."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import qsa_inputs as qi
from gpu_util import dev, k_dev, log

pytestmark = pytest.mark.gpu

import sparse_attention_block_qsa_amd as qsa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc(q32, kd, cfg, ids, vals, q_chunk=0):
    qts = cfg.G * cfg.H * cfg.D
    return qsa.lib.qsa_select_phase_noalloc(
        ctypes.c_void_p(q32.data_ptr()), None, qts, ctypes.c_void_p(kd.data_ptr()), kd.stride(0),
        ctypes.c_void_p(ids.data_ptr()), cfg.k, ctypes.c_void_p(vals.data_ptr()), cfg.G, cfg.nq,
        cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, q_chunk, 0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _reference(q32, kd, cfg, q_chunk):
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev(),
                            with_vals=True, q_chunk=q_chunk)
    ids, vals = qsa.select_phase(q32, kd, cfg.n_kv, cfg.bs, cfg.k, ws)
    return ids, vals


CASES = [
    # (config, q_chunk): the headline shape, then a smaller one; a prefill-like
    # shape of four KV heads that needs three passes through the 64 MiB array
    (qi.HEADLINE, 0), (qi.TINY, 0),
    (qi.Config("noalloc_chunks", 4, 4100, 8, 128, 2048 * 64 + 5, 64, 64, "normal", 4242), 0),
    (qi.CONFIGS["nq256_nkv4096"], 100),
]


def test_noalloc_matches_phase_two_calls_second_smaller():
    for cfg, q_chunk in [CASES[0], CASES[1]]:
        _check_case(cfg, q_chunk)


@pytest.mark.parametrize("case", CASES[2:], ids=lambda c: c[0].name)
def test_noalloc_matches_phase_chunked(case):
    _check_case(*case)


def _check_case(cfg, q_chunk):
    log(f"noalloc {cfg.name} q_chunk {q_chunk}")
    w = qi.make(cfg)
    q32 = torch.from_numpy(w.q32).to(dev())
    kd = k_dev(w.kblk)
    ids = torch.full((cfg.G, cfg.nq, cfg.k), -7, dtype=torch.int32, device=dev())
    vals = torch.full((cfg.G, cfg.nq, cfg.k), 7.0, dtype=torch.float32, device=dev())
    st = _noalloc(q32, kd, cfg, ids, vals, q_chunk)
    assert st == qsa.QSA_OK, qsa.status_string(st)
    row_bytes = 4 * cfg.G * (-(-max(cfg.nb, 1) // 32) * 32)
    fit = qsa.NOALLOC_SCRATCH_BYTES // row_bytes
    chunk = q_chunk if q_chunk else (0 if fit >= cfg.nq else fit)
    ref_ids, ref_vals = _reference(q32, kd, cfg, chunk)
    torch.cuda.synchronize()
    assert torch.equal(ids, ref_ids)
    assert torch.equal(vals.view(torch.int32), ref_vals.view(torch.int32))
    # a second call overwrites the same array: same bits again
    ids2 = torch.full_like(ids, -7)
    st = _noalloc(q32, kd, cfg, ids2, vals, q_chunk)
    assert st == qsa.QSA_OK
    torch.cuda.synchronize()
    assert torch.equal(ids2, ref_ids)
    # the one-pass phase (wide or small scorer) gives the same ids as any chunking
    if chunk:
        one_ids, _ = _reference(q32, kd, cfg, 0)
        torch.cuda.synchronize()
        assert torch.equal(ids, one_ids)


def test_noalloc_too_large_launches_nothing():
    cfg = qi.Config("noalloc_big", 4, 4096, 8, 128, 2048 * 64 + 5, 64, 64, "normal", 4243)
    q32 = torch.zeros((cfg.nq, cfg.G, cfg.H, cfg.D), dtype=torch.float32, device=dev())
    kd = torch.zeros((cfg.G, cfg.nb, cfg.D), dtype=torch.float16, device=dev())
    ids = torch.full((cfg.G, cfg.nq, cfg.k), -7, dtype=torch.int32, device=dev())
    vals = torch.full((cfg.G, cfg.nq, cfg.k), 7.0, dtype=torch.float32, device=dev())
    st = _noalloc(q32, kd, cfg, ids, vals, q_chunk=cfg.nq)
    assert st == qsa.QSA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert torch.all(ids == -7) and torch.all(vals == 7.0)
