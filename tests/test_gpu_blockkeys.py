"""GPU parity of qsa_block_keys (the block keys the scorer reads, built from
token keys) against the oracle, bit for bit: the mean of each block's token
keys, rounded once to the nearest fp16 (the reading taken for k_b, which
Strata pull request #228, part 1, indexes but does not define).  Write sets
are checked with canaries; the full-prefill shape is checked in full; a
phase over device-built keys equals one over the oracle's keys."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
from gpu_util import dev, guarded, log

pytestmark = pytest.mark.gpu

import sparse_attention_block_qsa_amd as qsa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tokens(rng, n, G, D, kind):
    if kind == "normal":
        return qi.f64_to_f16_bits(rng.standard_normal((n, G, D)) / np.sqrt(D))
    if kind == "wide":     # every finite exponent, subnormals, +-0, +-65504
        e = rng.integers(0, 31, (n, G, D))
        m = rng.integers(0, 1024, (n, G, D))
        s = rng.integers(0, 2, (n, G, D))
        bits = ((s << 15) | (e << 10) | m).astype(np.uint16)
        special = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x7BFF, 0xFBFF], np.uint16)
        pick = rng.random((n, G, D)) < 0.1
        bits[pick] = special[rng.integers(0, special.size, int(pick.sum()))]
        return bits
    assert kind == "ties"  # small integers: many means land on rounding ties
    return qi.f64_to_f16_bits(rng.integers(-3, 4, (n, G, D)) * 2.0 ** -24)


def _run(k_tok, n_kv, bs, tok_pad=0, nb_pad=0):
    """Device block keys through the C ABI with a padded token stride and a
    canary-guarded output of nb + nb_pad rows per head."""
    n, G, D = k_tok.shape
    nb = -(-n_kv // bs)
    row = G * D + tok_pad
    kt = torch.full((n, row), float("nan"), dtype=torch.float16, device=dev())
    kt[:, :G * D] = torch.from_numpy(k_tok.view(np.float16).reshape(n, G * D).copy()).to(dev())
    kt = kt.as_strided((n, G, D), (row, D, 1))
    # canaries in 32-bit units: each covers two fp16 keys
    out = guarded((G, max(nb, 1) + nb_pad, D // 2), torch.int32)
    qsa.block_keys(kt, n_kv, bs, out=out.view.view(torch.float16))
    torch.cuda.synchronize()
    m32 = np.zeros((G, max(nb, 1) + nb_pad, D // 2), dtype=bool)
    m32[:, :nb] = True
    assert out.outside_intact(m32) and out.written_all(m32), "block_keys write set"
    return out.view.view(torch.float16)[:, :nb].cpu().numpy().view(np.uint16)


CASES = [
    # (G, D, n_kv, bs, values, token pad)
    (1, 128, 64 * 7, 64, "normal", 0), (4, 128, 64 * 30 + 5, 64, "normal", 8),
    (3, 64, 1000, 64, "wide", 0), (2, 128, 333, 7, "wide", 16), (2, 64, 100, 3, "ties", 0),
    (1, 128, 97, 1, "wide", 0), (2, 64, 8192 * 2 + 100, 8192, "wide", 0),
    (5, 128, 40, 64, "ties", 24), (8, 64, 12345, 100, "normal", 0), (1, 64, 1, 64, "wide", 8),
]


@pytest.mark.parametrize("G,D,n_kv,bs,kind,tok_pad", CASES, ids=lambda v: str(v))
def test_block_keys_bit_exact(G, D, n_kv, bs, kind, tok_pad):
    rng = np.random.default_rng(7000 + G + D + n_kv + bs)
    k_tok = _tokens(rng, n_kv, G, D, kind)
    log(f"block keys G={G} D={D} n_kv={n_kv} bs={bs} {kind}")
    got = _run(k_tok, n_kv, bs, tok_pad=tok_pad, nb_pad=2)
    want = oracle.block_keys(k_tok, n_kv, bs)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} keys differ, first {bad[0]}: {got[tuple(bad[0])]:#06x} vs " \
                          f"{want[tuple(bad[0])]:#06x}"


def test_block_keys_empty_writes_nothing():
    k_tok = np.zeros((4, 2, 64), np.uint16)
    out = guarded((2, 3, 32), torch.int32)
    kt = torch.from_numpy(k_tok.view(np.float16)).to(dev())
    qsa.block_keys(kt, 0, 64, out=out.view.view(torch.float16))
    torch.cuda.synchronize()
    assert out.outside_intact(np.zeros((2, 3, 32), dtype=bool))


def test_block_keys_prefill_shape_and_phase():
    """4 KV heads x 131077 tokens (2048 blocks of 64 + a 5-token tail), D = 128:
    every key bit for bit; the phase over the device-built keys gives the same
    scores and ids as over the oracle's keys."""
    cfg = qi.PREFILL
    rng = np.random.default_rng(7100)
    k_tok = _tokens(rng, cfg.n_kv, cfg.G, cfg.D, "normal")
    kt = torch.from_numpy(k_tok.view(np.float16)).to(dev())
    kd = qsa.block_keys(kt, cfg.n_kv, cfg.bs)
    want = oracle.block_keys(k_tok, cfg.n_kv, cfg.bs)
    torch.cuda.synchronize()
    got = kd.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # a smaller query set over these keys, phase on both key sets
    q = torch.from_numpy(qi.make(cfg, with_q32=True).q32[:512]).to(dev())
    ws1 = qsa.PhaseWorkspace(512, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev())
    ws2 = qsa.PhaseWorkspace(512, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev())
    ids1 = qsa.select_phase(q, kd.contiguous(), cfg.n_kv, cfg.bs, cfg.k, ws1)
    ids2 = qsa.select_phase(q, torch.from_numpy(want.view(np.float16)).to(dev()), cfg.n_kv, cfg.bs,
                            cfg.k, ws2)
    torch.cuda.synchronize()
    assert torch.equal(ids1, ids2)
    nb = cfg.nb   # the workspace rows are padded past nb; only [0, nb) is written
    assert torch.equal(ws1.scores[:, :, :nb].view(torch.int32), ws2.scores[:, :, :nb].view(torch.int32))
