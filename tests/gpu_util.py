"""Helpers of the GPU parity tests: move seeded inputs to the device, call the
library through its C ABI with canary-guarded outputs, bring results back.

Canaries: every output buffer is a view into a larger allocation filled
with a sentinel NaN bit pattern; after a call, every element outside the
documented write set must still hold the sentinel (the pages assert the
scorer's write set with canaries: Strata pull request #228, part 1, parity
suite paragraph)."""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

import qsa_inputs as qi

SENTINEL = np.int32(0x7FBADBAD)   # a NaN no kernel produces
GUARD = 4096


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev() -> torch.device:
    return torch.device("cuda:0")


def q_dev(q16: np.ndarray, tok_pad: int = 0) -> torch.Tensor:
    """[nq, G, H, D] fp16 on device; tok_pad extra elements between tokens."""
    nq, G, H, D = q16.shape
    if tok_pad == 0:
        return torch.from_numpy(q16.view(np.float16).copy()).to(dev())
    row = G * H * D + tok_pad
    buf = torch.full((nq, row), float("nan"), dtype=torch.float16, device=dev())
    buf[:, :G * H * D] = torch.from_numpy(q16.view(np.float16).reshape(nq, -1).copy()).to(dev())
    return buf.as_strided((nq, G, H, D), (row, H * D, D, 1))


def k_dev(kblk: np.ndarray, nb_pad: int = 0) -> torch.Tensor:
    """[G, nb, D] fp16 on device; nb_pad extra (NaN) block rows per KV head."""
    G, nb, D = kblk.shape
    buf = torch.full((G, nb + nb_pad, D), float("nan"), dtype=torch.float16, device=dev())
    buf[:, :nb] = torch.from_numpy(kblk.view(np.float16).copy()).to(dev())
    return buf


@dataclass
class Guarded:
    flat: torch.Tensor      # int32 view of the whole allocation
    view: torch.Tensor      # the output view handed to the library
    off: int
    n: int

    def outside_intact(self, write_mask: np.ndarray) -> bool:
        """write_mask: bool over the view's elements (True = may be written)."""
        allv = self.flat.cpu().numpy()
        inside = allv[self.off:self.off + self.n].reshape(write_mask.shape)
        if np.any(allv[:self.off] != SENTINEL) or np.any(allv[self.off + self.n:] != SENTINEL):
            return False
        return bool(np.all(inside[~write_mask] == SENTINEL))

    def written_all(self, write_mask: np.ndarray) -> bool:
        inside = self.flat.cpu().numpy()[self.off:self.off + self.n].reshape(write_mask.shape)
        return not np.any(inside[write_mask] == SENTINEL)


def guarded(shape: tuple, dtype: torch.dtype) -> Guarded:
    n = int(np.prod(shape))
    flat = torch.full((GUARD + n + GUARD,), int(SENTINEL), dtype=torch.int32, device=dev())
    v = flat[GUARD:GUARD + n].view(dtype).view(shape)
    return Guarded(flat, v, GUARD, n)


def scores_mask(G: int, nq: int, ld: int, nb: int) -> np.ndarray:
    m = np.zeros((G, nq, ld), dtype=bool)
    m[:, :, :nb] = True
    return m


def run_block_scores(q16: np.ndarray, kblk: np.ndarray, n_kv: int, bs: int, *, ld_pad: int = 3,
                     tok_pad: int = 0, nb_pad: int = 0):
    """Returns (scores float64 [G*nq][nb], canaries intact, every cell written)."""
    import sparse_attention_block_qsa_amd as qsa
    nq, G, H, D = q16.shape
    nb = qi.Config("x", G, nq, H, D, n_kv, bs, 1, "normal", 0).nb
    ld = max(nb, 1) + ld_pad
    out = guarded((G, nq, ld), torch.float32)
    qd = q_dev(q16, tok_pad)
    kd = k_dev(kblk[:, :max(nb, 1)] if kblk.shape[1] >= max(nb, 1) else kblk, nb_pad)
    qsa.block_scores(qd, kd, n_kv, bs, out=out.view)
    torch.cuda.synchronize()
    mask = scores_mask(G, nq, ld, nb)
    intact = out.outside_intact(mask)
    written = out.written_all(mask)
    s = out.view[:, :, :nb].cpu().numpy().reshape(G * nq, nb).astype(np.float64)
    return s, intact, written
