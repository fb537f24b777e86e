"""QSA block-score select phase on MI355X (gfx950): thin Python binding.

Every step of the phase runs in the HIP kernels of libqsa.so (built from
``csrc/``; C ABI in ``include/qsa.h``).  This module only marshals arguments:
it takes torch tensors for device memory, passes their data pointers,
strides and torch's current HIP stream, and raises on a non-OK status.  There
is no CPU path: if the library is missing, importing this package fails.

    score(g, t, b) = sum_h relu( sum_i k[g, b, i] * q[t, g, h, i] )

(Strata pull request #228, part 1, score formula), then per (g, t) the top-k
blocks by (score descending, block id ascending).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_OK, QSA_ERR_ARG, QSA_ERR_UNSUPPORTED, QSA_ERR_HIP, QSA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
MAX_K = 64
NOALLOC_SCRATCH_BYTES = 64 << 20   # qsa.h QSA_NOALLOC_SCRATCH_BYTES
ABI_VERSION = 7   # qsa.h QSA_ABI_VERSION this binding is written for
BLOCK_KEYS_MAX_BS = 8192   # qsa.h QSA_BLOCK_KEYS_MAX_BS
FORCE_TAIL = 1   # qsa.h QSA_FORCE_TAIL
FUSED_SELECT = 2   # qsa.h QSA_FUSED_SELECT
STREAM_SELECT = 4   # qsa.h QSA_STREAM_SELECT
EXPORTS = ("qsa_abi_version", "qsa_status_string", "qsa_convert_f32_f16", "qsa_block_keys",
           "qsa_block_scores", "qsa_select_topk", "qsa_select_phase", "qsa_select_phase_noalloc",
           "qsa_sparse_attention", "qsa_sparse_attention_ws_floats")


class QSAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    L.qsa_abi_version.restype = ctypes.c_int
    L.qsa_status_string.argtypes = [ctypes.c_int]
    L.qsa_status_string.restype = ctypes.c_char_p
    L.qsa_convert_f32_f16.argtypes = [vp, vp, i64, vp]
    L.qsa_convert_f32_f16.restype = ctypes.c_int
    L.qsa_block_keys.argtypes = [vp, i64, vp, i64, i32, i32, i64, i32, vp]
    L.qsa_block_keys.restype = ctypes.c_int
    L.qsa_sparse_attention.argtypes = [vp, i64, vp, vp, i64, vp, i64, vp, i64, i32, i32, i32, i32,
                                       i64, i32, i32, vp, i64, vp]
    L.qsa_sparse_attention.restype = ctypes.c_int
    L.qsa_sparse_attention_ws_floats.argtypes = [i32, i32, i32, i32, i32, i32]
    L.qsa_sparse_attention_ws_floats.restype = ctypes.c_int64
    L.qsa_block_scores.argtypes = [vp, i64, vp, i64, vp, i64, i32, i32, i32, i32, i64, i32, u32,
                                   vp]
    L.qsa_block_scores.restype = ctypes.c_int
    L.qsa_select_topk.argtypes = [vp, i64, i64, i32, i32, vp, i64, vp, vp]
    L.qsa_select_topk.restype = ctypes.c_int
    L.qsa_select_phase.argtypes = [vp, vp, i64, vp, i64, vp, i64, vp, i64, vp, i32, i32, i32,
                                   i32, i64, i32, i32, i64, u32, vp]
    L.qsa_select_phase.restype = ctypes.c_int
    L.qsa_select_phase_noalloc.argtypes = [vp, vp, i64, vp, i64, vp, i64, vp, i32, i32, i32, i32,
                                           i64, i32, i32, i64, u32, vp]
    L.qsa_select_phase_noalloc.restype = ctypes.c_int
    if L.qsa_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH}: ABI version {L.qsa_abi_version()}, this binding needs "
                          f"{ABI_VERSION}; rebuild with __graft_entry__.build()")
    return L


lib = _load()


def status_string(st: int) -> str:
    return lib.qsa_status_string(st).decode()


def _check(fn: str, st: int) -> None:
    if st != QSA_OK:
        raise QSAError(fn, st, status_string(st))


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream: torch.cuda.Stream | None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def n_blocks(n_kv: int, bs: int) -> int:
    return -(-n_kv // bs)


def _check_q(q: torch.Tensor, dtype) -> tuple[int, int, int, int, int]:
    if q.dim() != 4 or q.dtype != dtype or not q.is_cuda:
        raise ValueError(f"queries must be a 4-D {dtype} CUDA tensor [nq, G, H, D]")
    nq, G, H, D = q.shape
    if q.stride(3) != 1 or q.stride(2) != D or q.stride(1) != H * D:
        raise ValueError("queries: the (G, H, D) dims must be contiguous")
    return nq, G, H, D, q.stride(0)


def _check_k(kblk: torch.Tensor, G: int, D: int, nb: int) -> int:
    if (kblk.dim() != 3 or kblk.dtype != torch.float16 or not kblk.is_cuda or kblk.shape[0] != G
            or kblk.shape[2] != D or kblk.shape[1] < nb):
        raise ValueError("kblk must be a float16 CUDA tensor [G, >= nb, D]")
    if kblk.stride(2) != 1 or kblk.stride(1) != D:
        raise ValueError("kblk: the (nb, D) dims must be contiguous")
    return kblk.stride(0)


def _scores_view(out: torch.Tensor, G: int, nq: int, nb: int) -> int:
    if out.dim() != 3 or out.dtype != torch.float32 or tuple(out.shape[:2]) != (G, nq) \
            or out.shape[2] < nb or out.stride(2) != 1 or (nq > 1 and out.stride(0) != nq * out.stride(1)):
        raise ValueError("scores must be float32 [G, nq, >= nb] with rows at a common stride")
    return out.stride(1)


def convert_f32_f16(src: torch.Tensor, out: torch.Tensor | None = None,
                    stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """fp32 -> fp16 (round to nearest even) over a contiguous tensor."""
    if src.dtype != torch.float32 or not src.is_contiguous() or not src.is_cuda:
        raise ValueError("src must be a contiguous float32 CUDA tensor")
    if out is None:
        out = torch.empty(src.shape, dtype=torch.float16, device=src.device)
    if out.dtype != torch.float16 or not out.is_contiguous() or out.numel() != src.numel():
        raise ValueError("out must be a contiguous float16 tensor of src's size")
    _check("qsa_convert_f32_f16",
           lib.qsa_convert_f32_f16(_ptr(src), _ptr(out), src.numel(), _stream(stream)))
    return out


def block_keys(k_tok: torch.Tensor, n_kv: int, bs: int, out: torch.Tensor | None = None,
               stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Block keys [G, nb, D] fp16 from token keys k_tok [>= n_kv, G, D] fp16
    (token-major, the (G, D) dims contiguous): the mean of each block's
    tokens rounded once to fp16 (a view of ``out`` when given)."""
    if k_tok.dim() != 3 or k_tok.dtype != torch.float16 or not k_tok.is_cuda \
            or k_tok.shape[0] < n_kv or k_tok.stride(2) != 1 or k_tok.stride(1) != k_tok.shape[2]:
        raise ValueError("k_tok must be a float16 CUDA tensor [>= n_kv, G, D], (G, D) contiguous")
    _, G, D = k_tok.shape
    nb = n_blocks(n_kv, bs)
    if out is None:
        out = torch.empty((G, max(nb, 1), D), dtype=torch.float16, device=k_tok.device)
    if out.dim() != 3 or out.dtype != torch.float16 or out.shape[0] != G or out.shape[1] < nb \
            or out.shape[2] != D or out.stride(2) != 1 or out.stride(1) != D:
        raise ValueError("out must be float16 [G, >= nb, D] with (nb, D) contiguous")
    _check("qsa_block_keys",
           lib.qsa_block_keys(_ptr(k_tok), k_tok.stride(0), _ptr(out), out.stride(0), G, D, n_kv,
                              bs, _stream(stream)))
    return out[:, :nb]


def block_scores(q16: torch.Tensor, kblk: torch.Tensor, n_kv: int, bs: int,
                 out: torch.Tensor | None = None, force_tail: bool = False,
                 stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Scores [G, nq, nb] (a view of ``out`` when given, whose last dim may be
    longer than nb: only [..., :nb] is written).  force_tail: the partial
    last block's score gets 1e9 added (FORCE_TAIL)."""
    nq, G, H, D, qts = _check_q(q16, torch.float16)
    nb = n_blocks(n_kv, bs)
    khs = _check_k(kblk, G, D, nb)
    if out is None:
        out = torch.empty((G, nq, max(nb, 1)), dtype=torch.float32, device=q16.device)
    ld_s = _scores_view(out, G, nq, nb)
    _check("qsa_block_scores",
           lib.qsa_block_scores(_ptr(q16), qts, _ptr(kblk), khs, _ptr(out), ld_s, G, nq, H, D,
                                n_kv, bs, FORCE_TAIL if force_tail else 0, _stream(stream)))
    return out[..., :nb]


def select_topk(scores: torch.Tensor, nb: int, k: int, ids: torch.Tensor | None = None,
                vals: torch.Tensor | None = None, want_vals: bool = False,
                stream: torch.cuda.Stream | None = None):
    """Top-k ids per row of a 2-D float32 [rows, >= nb] score matrix.
    Returns ids [rows, k] (int32, -1 padded) or (ids, vals)."""
    if scores.dim() != 2 or scores.dtype != torch.float32 or scores.stride(1) != 1 \
            or scores.shape[1] < nb:
        raise ValueError("scores must be float32 [rows, >= nb] with unit column stride")
    rows = scores.shape[0]
    if ids is None:
        ids = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    if want_vals and vals is None:
        vals = torch.empty((rows, k), dtype=torch.float32, device=scores.device)
    if ids.dim() != 2 or ids.dtype != torch.int32 or ids.stride(1) != 1 or ids.shape[0] != rows \
            or ids.shape[1] < k:
        raise ValueError("ids must be int32 [rows, >= k] with unit column stride")
    if vals is not None and (vals.dtype != torch.float32 or vals.stride() != ids.stride()
                             or vals.shape != ids.shape):
        raise ValueError("vals must be float32 with the layout of ids")
    _check("qsa_select_topk",
           lib.qsa_select_topk(_ptr(scores), scores.stride(0), rows, nb, k, _ptr(ids),
                               ids.stride(0), _ptr(vals), _stream(stream)))
    return (ids, vals) if (want_vals or vals is not None) else ids


class PhaseWorkspace:
    """Device buffers of one select phase, allocated once and reused for
    phases of exactly this geometry (select_phase refuses any other).  With
    keep_q16 the phase also stores the fp16 conversion of fp32 queries in q16
    (one more write of the queries); without it q16 is None and the scorers
    convert the queries in registers only.  With 0 < q_chunk < nq the score
    workspace holds G*q_chunk rows and the phase walks the queries in chunks
    of q_chunk."""

    def __init__(self, nq: int, G: int, H: int, D: int, n_kv: int, bs: int, k: int,
                 device="cuda", q_chunk: int = 0, with_vals: bool = False, ld_pad: int = 0,
                 keep_q16: bool = False):
        if q_chunk < 0:
            raise ValueError("q_chunk must be >= 0")
        self.geometry = (nq, G, H, D, n_kv, bs, k)
        self.nb = n_blocks(n_kv, bs)
        qc = q_chunk if 0 < q_chunk < nq else nq
        self.q_chunk = q_chunk
        self.chunk_rows = qc
        # Rows start on 128-byte boundaries: every 32-column tile store of the
        # scorer then fills whole cache lines.
        self.ld_s = -(-(max(self.nb, 1) + ld_pad) // 32) * 32
        self.scores = torch.empty((G, qc, self.ld_s), dtype=torch.float32, device=device)
        self.q16 = (torch.empty((nq, G, H, D), dtype=torch.float16, device=device)
                    if keep_q16 else None)
        self.ids = torch.empty((G, nq, k), dtype=torch.int32, device=device)
        self.vals = torch.empty((G, nq, k), dtype=torch.float32, device=device) if with_vals else None


def select_phase(q: torch.Tensor, kblk: torch.Tensor, n_kv: int, bs: int, k: int,
                 ws: PhaseWorkspace | None = None, q_chunk: int | None = None,
                 force_tail: bool = False, fused_select: bool = False,
                 stream_select: bool = False, stream: torch.cuda.Stream | None = None):
    """The whole phase: (fp32 -> fp16 conversion when q is float32), scores,
    top-k.  Returns ids [G, nq, k] (and vals when the workspace has them).
    fp32 queries are converted by the scorers as they load them; without a
    kept fp16 copy (ws.q16 is None) their rows must be 16-byte aligned, which
    a contiguous tensor from the caching allocator always is.  q_chunk is the
    workspace's when one is given (a different value is refused), else 0.
    force_tail: the forced-tail rule (FORCE_TAIL); fused_select: select inside
    the scorer's launch where the fused scorer serves the shape (FUSED_SELECT),
    with the same results; stream_select: keep a running selection per row
    while the scores stream by, writing no score, where the streaming scorer
    serves the shape (STREAM_SELECT; ws.scores is then left untouched), with
    the same results."""
    fp32 = q.dtype == torch.float32
    nq, G, H, D, qts = _check_q(q, torch.float32 if fp32 else torch.float16)
    if fp32 and not q.is_contiguous():
        raise ValueError("fp32 queries must be contiguous")
    nb = n_blocks(n_kv, bs)
    khs = _check_k(kblk, G, D, nb)
    if ws is None:
        ws = PhaseWorkspace(nq, G, H, D, n_kv, bs, k, q.device, q_chunk or 0)
    else:
        if ws.geometry != (nq, G, H, D, n_kv, bs, k):
            raise ValueError(f"workspace built for (nq, G, H, D, n_kv, bs, k) = {ws.geometry}, "
                             f"called with {(nq, G, H, D, n_kv, bs, k)}")
        if q_chunk is not None and q_chunk != ws.q_chunk:
            raise ValueError(f"q_chunk {q_chunk} differs from the workspace's {ws.q_chunk}")
    q16 = ws.q16 if fp32 else q
    if fp32 and q16 is not None and q16.stride(0) != qts:
        raise ValueError("workspace q16 layout does not match the queries")
    _check("qsa_select_phase",
           lib.qsa_select_phase(_ptr(q) if fp32 else None, _ptr(q16), qts, _ptr(kblk), khs,
                                _ptr(ws.scores), ws.ld_s, _ptr(ws.ids), ws.ids.stride(1),
                                _ptr(ws.vals), G, nq, H, D, n_kv, bs, k, ws.q_chunk,
                                (FORCE_TAIL if force_tail else 0) |
                                (FUSED_SELECT if fused_select else 0) |
                                (STREAM_SELECT if stream_select else 0), _stream(stream)))
    return (ws.ids, ws.vals) if ws.vals is not None else ws.ids


def select_phase_noalloc(q: torch.Tensor, kblk: torch.Tensor, n_kv: int, bs: int, k: int,
                         ids: torch.Tensor, vals: torch.Tensor | None = None, q_chunk: int = 0,
                         q16: torch.Tensor | None = None, force_tail: bool = False,
                         stream_select: bool = False, stream: torch.cuda.Stream | None = None):
    """The whole phase with no device allocation: scores go to the library's
    fixed per-GPU scratch array (NOALLOC_SCRATCH_BYTES), ids [G, nq, k] and
    optional vals are the caller's.  q is float32 (with an optional fp16
    buffer q16 that receives the converted queries) or float16.
    stream_select as select_phase (the shapes it serves leave the scratch
    array untouched)."""
    fp32 = q.dtype == torch.float32
    nq, G, H, D, qts = _check_q(q, torch.float32 if fp32 else torch.float16)
    nb = n_blocks(n_kv, bs)
    khs = _check_k(kblk, G, D, nb)
    if ids.dtype != torch.int32 or tuple(ids.shape) != (G, nq, k) or ids.stride(2) != 1 \
            or ids.stride(0) != nq * ids.stride(1):
        raise ValueError("ids must be int32 [G, nq, k] with rows at a common stride")
    if vals is not None and (vals.dtype != torch.float32 or vals.shape != ids.shape
                             or vals.stride() != ids.stride()):
        raise ValueError("vals must be float32 with the layout of ids")
    qsrc16 = q16 if fp32 else q
    if fp32 and q16 is not None and (q16.dtype != torch.float16 or q16.stride(0) != qts):
        raise ValueError("q16 must be float16 with the queries' layout")
    _check("qsa_select_phase_noalloc",
           lib.qsa_select_phase_noalloc(_ptr(q) if fp32 else None, _ptr(qsrc16), qts, _ptr(kblk),
                                        khs, _ptr(ids), ids.stride(1), _ptr(vals), G, nq, H, D,
                                        n_kv, bs, k, q_chunk,
                                        (FORCE_TAIL if force_tail else 0) |
                                        (STREAM_SELECT if stream_select else 0), _stream(stream)))
    return (ids, vals) if vals is not None else ids


def attention_workspace(G: int, nq: int, H: int, D: int, bs: int, k: int,
                        device="cuda") -> torch.Tensor | None:
    """The workspace that lets sparse_attention split few rows over several
    workgroups (None when it would not split them)."""
    n = lib.qsa_sparse_attention_ws_floats(G, nq, H, D, bs, k)
    return torch.empty(n, dtype=torch.float32, device=device) if n > 0 else None


def sparse_attention(q16: torch.Tensor, k_tok: torch.Tensor, v_tok: torch.Tensor,
                     ids: torch.Tensor, n_kv: int, bs: int, out: torch.Tensor | None = None,
                     ws: torch.Tensor | None | bool = True,
                     stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Attention of every query head over the tokens of its row's selected
    blocks: q16 [nq, G, H, D] fp16, k_tok / v_tok [>= n_kv, G, D] fp16
    (token-major), ids [G, nq, k] int32 (the selector's ids, -1 = empty).
    ws: a workspace tensor, None (no row splitting) or True (allocate the
    one attention_workspace gives).  Returns out [nq, G, H, D] float32."""
    nq, G, H, D, qts = _check_q(q16, torch.float16)
    for name, kv in (("k_tok", k_tok), ("v_tok", v_tok)):
        if kv.dim() != 3 or kv.dtype != torch.float16 or not kv.is_cuda or kv.shape[0] < n_kv \
                or tuple(kv.shape[1:]) != (G, D) or kv.stride(2) != 1 or kv.stride(1) != D:
            raise ValueError(f"{name} must be float16 [>= n_kv, G, D] with (G, D) contiguous")
    if k_tok.stride(0) != v_tok.stride(0):
        raise ValueError("k_tok and v_tok must share their token stride")
    if ids.dim() != 3 or ids.dtype != torch.int32 or tuple(ids.shape[:2]) != (G, nq) \
            or ids.stride(2) != 1 or (nq > 1 and ids.stride(0) != nq * ids.stride(1)):
        raise ValueError("ids must be int32 [G, nq, k] with rows at a common stride")
    k = ids.shape[2]
    if out is None:
        out = torch.empty((nq, G, H, D), dtype=torch.float32, device=q16.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (nq, G, H, D) or out.stride(3) != 1 \
            or out.stride(2) != D or out.stride(1) != H * D:
        raise ValueError("out must be float32 [nq, G, H, D] with (G, H, D) contiguous")
    if ws is True:
        ws = attention_workspace(G, nq, H, D, bs, k, q16.device)
    if ws is not None and (ws.dtype != torch.float32 or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous float32 tensor")
    _check("qsa_sparse_attention",
           lib.qsa_sparse_attention(_ptr(q16), qts, _ptr(k_tok), _ptr(v_tok), k_tok.stride(0),
                                    _ptr(ids), ids.stride(1), _ptr(out), out.stride(0), G, nq, H,
                                    D, n_kv, bs, k, _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(stream)))
    return out
