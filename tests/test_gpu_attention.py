"""GPU parity of qsa_sparse_attention (attention of every query head over
the tokens of its row's selected blocks, the step after the selection)
against the float64 oracle: every output element within the oracle's bound
B of an fp32 computation, +2.5*B perturbations failing the same check, exact
write sets, and rows without a selected token giving 0.  The ids come from
the library's own selection phase, or are drawn at random with empty slots."""
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


def _kv(rng, n_kv, G, D, scale=1.0):
    n = max(n_kv, 1)
    k = qi.f64_to_f16_bits(rng.standard_normal((n, G, D)) * scale)
    v = qi.f64_to_f16_bits(rng.standard_normal((n, G, D)))
    return k, v


def _run(q16, kt, vt, ids, n_kv, bs, tok_pad=0, split=True):
    nq, G, H, D = q16.shape
    row = G * H * D + tok_pad
    out = guarded((nq, row), torch.float32)
    qd = torch.from_numpy(q16.view(np.float16)).to(dev())
    kd = torch.from_numpy(kt.view(np.float16)).to(dev())
    vd = torch.from_numpy(vt.view(np.float16)).to(dev())
    idd = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev())
    view = out.view.as_strided((nq, G, H, D), (row, H * D, D, 1))
    ws = qsa.attention_workspace(G, nq, H, D, bs, ids.shape[2], dev()) if split else None
    st = qsa.lib.qsa_sparse_attention(qsa._ptr(qd), G * H * D, qsa._ptr(kd), qsa._ptr(vd), G * D,
                                      qsa._ptr(idd), ids.shape[2], qsa._ptr(view), row, G, nq, H,
                                      D, n_kv, bs, ids.shape[2], qsa._ptr(ws),
                                      0 if ws is None else ws.numel(), qsa._stream(None))
    assert st == qsa.QSA_OK, qsa.status_string(st)
    torch.cuda.synchronize()
    mask = np.zeros((nq, row), dtype=bool)
    mask[:, :G * H * D] = True
    assert out.outside_intact(mask) and out.written_all(mask), "attention write set"
    return view.cpu().numpy().astype(np.float64)


def _check(o, q16, kt, vt, ids, n_kv, bs, name):
    ref, B = oracle.attention(q16, kt, vt, ids, n_kv, bs)
    res = oracle.check_attention(o, ref, B)
    log(f"  [{name}] {res}")
    assert res.ok, f"{name}: {res}"
    if np.any(B > 0):
        assert not oracle.check_attention(o + 2.5 * B, ref, B).ok
        i = np.flatnonzero(B.ravel() > 0)[0]
        o2 = o.copy().ravel()
        o2[i] = ref.ravel()[i] + 2.5 * B.ravel()[i]
        assert not oracle.check_attention(o2.reshape(o.shape), ref, B).ok


# (name, G, nq, H, D, n_kv, bs, k, q scale): the pages' configurations' shapes
# and ragged ones (odd H, blocks not multiples of 64, a partial last block)
RANDOM = [
    ("tiny", 1, 37, 4, 64, 1000, 64, 4, 1.0), ("c2", 1, 64, 8, 128, 4096, 64, 16, 0.09),
    ("odd_h", 2, 9, 3, 128, 2000, 100, 8, 0.3), ("h12_d64", 3, 7, 12, 64, 777, 32, 12, 0.5),
    ("h16", 1, 5, 16, 128, 640, 64, 10, 0.2), ("h1_bs200", 2, 11, 1, 64, 5000, 200, 9, 1.0),
    ("big_logits", 1, 6, 8, 128, 3000, 64, 20, 1.5),
    # blocks of several chunks with a ragged last one at D = 128 (the
    # weighted values on the matrix cores, two passes per chunk), 5 and 6
    # heads (padded columns)
    ("d128_bs200_h6", 2, 7, 6, 128, 5003, 200, 9, 0.8), ("d128_bs100_h5", 1, 10, 5, 128, 3001, 100, 12, 1.0),
    ("d64_bs130_h8", 1, 8, 8, 64, 2600, 130, 10, 1.0),
]


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: c[0])
def test_attention_random_ids_within_bound(case):
    name, G, nq, H, D, n_kv, bs, k, qscale = case
    rng = np.random.default_rng(8000 + G * 100 + H * 10 + D)
    log(f"attention {case}")
    q16 = qi.f64_to_f16_bits(rng.standard_normal((nq, G, H, D)) * qscale)
    kt, vt = _kv(rng, n_kv, G, D)
    nb = -(-n_kv // bs)
    ids = np.full((G, nq, k), -1, np.int32)
    for g in range(G):
        for t in range(nq):
            sel = rng.permutation(nb)[:min(k, nb)]
            ids[g, t, :sel.size] = sel
            if t % 5 == 1:
                ids[g, t, ::2] = -1                # empty slots between real ones
            if t % 7 == 3:
                ids[g, t, 0] = nb - 1              # the partial last block
    if nq > 4:
        ids[:, 4] = -1                             # rows with no token at all
    for split in (True, False):   # rows over several workgroups, or one each
        o = _run(q16, kt, vt, ids, n_kv, bs, tok_pad=8, split=split)
        if nq > 4:
            assert np.all(o[4] == 0)
        _check(o, q16, kt, vt, ids, n_kv, bs, f"{name} split={split}")


def test_attention_nkv0_gives_zeros():
    rng = np.random.default_rng(8100)
    q16 = qi.f64_to_f16_bits(rng.standard_normal((5, 2, 4, 64)))
    kt, vt = _kv(rng, 0, 2, 64)
    ids = np.full((2, 5, 4), -1, np.int32)
    o = _run(q16, kt, vt, ids, 0, 64)
    assert np.all(o == 0)


@pytest.mark.parametrize("cfg_name", ["nq256_nkv32768", "nq256_nkv131072", "decode_g8_nq1_nkv131109"])
def test_attention_over_phase_selection(cfg_name):
    """The selection phase's own ids (k = 32 / 64 of 512 / 2048+ blocks)."""
    cfg = qi.CONFIGS[cfg_name]
    rng = np.random.default_rng(8200)
    w = qi.make(cfg)
    kt, vt = _kv(rng, cfg.n_kv, cfg.G, cfg.D)
    ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev())
    ids = qsa.select_phase(torch.from_numpy(w.q32).to(dev()),
                           torch.from_numpy(w.kblk.view(np.float16)).to(dev()), cfg.n_kv,
                           cfg.bs, cfg.k, ws)
    torch.cuda.synchronize()
    ids_np = ids.cpu().numpy()
    log(f"attention over the phase's selection, {cfg_name}")
    o = _run(w.q16, kt, vt, ids_np, cfg.n_kv, cfg.bs)
    _check(o, w.q16, kt, vt, ids_np, cfg.n_kv, cfg.bs, cfg_name)
