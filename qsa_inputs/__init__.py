"""Seeded synthetic inputs for the QSA block-score select phase.

This module is shared by the test suite, the oracle checks and the benchmark.
It holds no arithmetic of the method itself: it only draws random numbers,
shapes them into the query / block-key tensors and rounds them to fp16 bits.

Workloads (shapes and value distributions follow the QSA select workloads the
Strata pull requests #228 and #856 describe: nq = 256 queries against 1K-128K
tokens of context, plus a full-prefill query chunk):

    name                          G  nq     H  D    n_kv    bs  k   values
    tiny_nq37_nkv1000             1  37     4  64   1000    64  4   U(-1,1)
    nq256_nkv4096                 1  256    8  128  4096    64  16  N(0,1)/sqrt(D)
    nq256_nkv32768                1  256    8  128  32768   64  32  N(0,1)/sqrt(D)
    nq256_nkv131072               1  256    8  128  131072  64  64  N(0,1)/sqrt(D)
    prefill_g4_nq16384_nkv131077  4  16384  8  128  131077  64  64  N(0,1)/sqrt(D)

Random stream: splitmix64 in counter form. For a tensor with tag ``tag`` the
state starts at ``seed ^ (tag * 0x9E3779B97F4A7C15)`` and draw i (0-based) is
the splitmix64 finaliser applied to ``state + (i + 1) * 0x9E3779B97F4A7C15``
(mod 2^64), so any slice of a stream can be produced on its own.
Uniform draws are ``(x >> 11) * 2^-53``; normals are Box-Muller pairs in f64;
values are scaled in f64 and rounded once, directly from f64 to fp16
(round to nearest even), so there is no double rounding.

Layouts (all row-major):
    q16   uint16 [nq][G][H][D]   fp16 bits; head (g, h) of token t
    kblk  uint16 [G][nb][D]      fp16 bits; one key vector per KV block
    q32   float32 [nq][G][H][D]  the exact widening of q16 (or, for the
                                 conversion fixture, values that are not
                                 fp16-exact)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
TAG_Q = 1
TAG_K = 2
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    """splitmix64 finaliser (Steele, Lea, Flood 2014), elementwise on uint64."""
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, tag: int, start: int, count: int) -> np.ndarray:
    """Draws [start, start + count) of the (seed, tag) stream as uint64."""
    state = np.uint64((seed ^ ((tag * 0x9E3779B97F4A7C15) & (2**64 - 1))) & (2**64 - 1))
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(state + idx * GAMMA)


def uniform01(seed: int, tag: int, start: int, count: int) -> np.ndarray:
    x = splitmix64(seed, tag, start, count)
    return (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, tag: int, n: int) -> np.ndarray:
    """n standard normals: Box-Muller on consecutive uniform pairs."""
    out = np.empty(n, dtype=np.float64)
    npairs = (n + 1) // 2
    for p0 in range(0, npairs, _CHUNK):
        p1 = min(npairs, p0 + _CHUNK)
        u = uniform01(seed, tag, 2 * p0, 2 * (p1 - p0))
        u1, u2 = u[0::2], u[1::2]
        r = np.sqrt(-2.0 * np.log1p(-u1))  # 1 - u1 lies in (0, 1]
        th = (2.0 * math.pi) * u2
        pair = np.empty(2 * (p1 - p0), dtype=np.float64)
        pair[0::2] = r * np.cos(th)
        pair[1::2] = r * np.sin(th)
        lo, hi = 2 * p0, min(n, 2 * p1)
        out[lo:hi] = pair[: hi - lo]
    return out


def uniform_pm1(seed: int, tag: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, _CHUNK):
        c = min(_CHUNK, n - s)
        out[s : s + c] = 2.0 * uniform01(seed, tag, s, c) - 1.0
    return out


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round f64 -> fp16 (nearest even, directly from f64) and return the bits."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of fp16 bits to float32."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


@dataclass(frozen=True)
class Config:
    name: str
    G: int
    nq: int
    H: int
    D: int
    n_kv: int
    bs: int
    k: int
    dist: str  # "uniform" (U(-1,1)) or "normal" (N(0,1)/sqrt(D))
    seed: int

    @property
    def nb(self) -> int:
        return -(-self.n_kv // self.bs)

    @property
    def nf(self) -> int:
        return self.n_kv // self.bs

    @property
    def rows(self) -> int:
        return self.G * self.nq

    @property
    def flop(self) -> int:
        """2*H*D multiply-adds per (query, KV head, block) cell."""
        return 2 * self.rows * self.H * self.D * self.nb


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny_nq37_nkv1000", 1, 37, 4, 64, 1000, 64, 4, "uniform", 1001),
        Config("nq256_nkv4096", 1, 256, 8, 128, 4096, 64, 16, "normal", 1002),
        Config("nq256_nkv32768", 1, 256, 8, 128, 32768, 64, 32, "normal", 1003),
        Config("nq256_nkv131072", 1, 256, 8, 128, 131072, 64, 64, "normal", 1004),
        Config("prefill_g4_nq16384_nkv131077", 4, 16384, 8, 128, 131077, 64, 64, "normal", 1005),
        # one decode step: one query per KV head of a GQA layer with 64 query
        # heads, 128K tokens plus a partial block
        Config("decode_g8_nq1_nkv131109", 8, 1, 8, 128, 131109, 64, 64, "normal", 1006),
    ]
}
TINY = CONFIGS["tiny_nq37_nkv1000"]
HEADLINE = CONFIGS["nq256_nkv131072"]
PREFILL = CONFIGS["prefill_g4_nq16384_nkv131077"]
DECODE = CONFIGS["decode_g8_nq1_nkv131109"]


@dataclass
class Workload:
    cfg: Config
    q16: np.ndarray          # uint16 [nq][G][H][D]
    kblk: np.ndarray         # uint16 [G][nb][D]
    q32: np.ndarray | None = None  # float32 [nq][G][H][D]
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_kv(self) -> int:
        return self.cfg.n_kv


def _draw(cfg: Config, tag: int, n: int, seed: int | None = None) -> np.ndarray:
    s = cfg.seed if seed is None else seed
    if cfg.dist == "uniform":
        return uniform_pm1(s, tag, n)
    if cfg.dist == "normal":
        return normal(s, tag, n) / math.sqrt(cfg.D)
    raise ValueError(cfg.dist)


def make(cfg: Config | str, *, n_kv: int | None = None, with_q32: bool = True) -> Workload:
    """The seeded workload of a config. ``n_kv`` overrides the context length
    (the key table keeps at least one block so that it has a valid pointer)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if n_kv is not None:
        cfg = Config(cfg.name + f"_nkv{n_kv}", cfg.G, cfg.nq, cfg.H, cfg.D, n_kv,
                     cfg.bs, cfg.k, cfg.dist, cfg.seed)
    nq, G, H, D = cfg.nq, cfg.G, cfg.H, cfg.D
    nq_elems = nq * G * H * D
    q16 = f64_to_f16_bits(_draw(cfg, TAG_Q, nq_elems)).reshape(nq, G, H, D)
    nb_alloc = max(cfg.nb, 1)
    kblk = f64_to_f16_bits(_draw(cfg, TAG_K, G * nb_alloc * D)).reshape(G, nb_alloc, D)
    q32 = f16_bits_to_f32(q16) if with_q32 else None
    return Workload(cfg, q16, kblk, q32)


def scaled_by_8(w: Workload) -> Workload:
    """The same tensors multiplied by 8 (exact in fp16 while |x| < 8188)."""
    q = w.q16.view(np.float16).astype(np.float64) * 8.0
    k = w.kblk.view(np.float16).astype(np.float64) * 8.0
    q16 = f64_to_f16_bits(q)
    kb = f64_to_f16_bits(k)
    return Workload(w.cfg, q16, kb, f16_bits_to_f32(q16), note="x8")


def coded_fixture(cfg: Config) -> Workload:
    """One-hot / coordinate-coded adversarial fixture (no random draws).

    q[t, g, h, i] = 1 if i == c(t, h) else 0 with
        c(t, h) = band*h + (mix(t*H + h) mod band),   band = D // H,
    i.e. one channel per head inside the head's own band, so that a head
    mix-up, a transposed fragment or a duplicated lane moves the selected
    channel.  K[g, b, i] = (mix(b*D + i + g*2^40) mod 2039) - 1019, an integer
    that encodes (g, b, i) and has both signs.  Every score is then a sum of
    at most H integers of magnitude < 1020: exact in fp32 in any order.
    """
    nq, G, H, D = cfg.nq, cfg.G, cfg.H, cfg.D
    band = D // H
    assert band >= 1
    th = (np.arange(nq, dtype=np.uint64)[:, None] * np.uint64(H)
          + np.arange(H, dtype=np.uint64)[None, :])
    with np.errstate(over="ignore"):
        ch = (np.uint64(band) * np.arange(H, dtype=np.uint64)[None, :]
              + _mix(th) % np.uint64(band)).astype(np.int64)  # [nq][H]
    q = np.zeros((nq, G, H, D), dtype=np.float64)
    for h in range(H):
        q[np.arange(nq), :, h, ch[:, h]] = 1.0
    nb_alloc = max(cfg.nb, 1)
    gi = (np.arange(G, dtype=np.uint64)[:, None, None] << np.uint64(40))
    bi = np.arange(nb_alloc, dtype=np.uint64)[None, :, None] * np.uint64(D)
    ii = np.arange(D, dtype=np.uint64)[None, None, :]
    with np.errstate(over="ignore"):
        kv = (_mix(gi + bi + ii) % np.uint64(2039)).astype(np.int64) - 1019
    q16 = f64_to_f16_bits(q)
    kb = f64_to_f16_bits(kv.astype(np.float64))
    return Workload(cfg, q16, kb, f16_bits_to_f32(q16), note="coded",
                    extra={"channel": ch, "kint": kv})


def integer_fixture(cfg: Config, seed: int = 2002) -> Workload:
    """Dense fp16-exact integers: q ~ U{1..7}; k ~ U{-7..7} on even blocks and
    U{1..7} on odd blocks.  Dots reach a few thousand, so fp16 accumulation
    would lose odd integers, while fp32 holds every partial sum exactly."""
    nq, G, H, D = cfg.nq, cfg.G, cfg.H, cfg.D
    nb_alloc = max(cfg.nb, 1)
    xq = splitmix64(seed, TAG_Q, 0, nq * G * H * D)
    q = (xq % np.uint64(7)).astype(np.int64) + 1
    xk = splitmix64(seed, TAG_K, 0, G * nb_alloc * D)
    ke = (xk % np.uint64(15)).astype(np.int64) - 7
    ko = (xk % np.uint64(7)).astype(np.int64) + 1
    k = ke.reshape(G, nb_alloc, D)
    odd = (np.arange(nb_alloc) % 2 == 1)
    k[:, odd, :] = ko.reshape(G, nb_alloc, D)[:, odd, :]
    q16 = f64_to_f16_bits(q.reshape(nq, G, H, D).astype(np.float64))
    kb = f64_to_f16_bits(k.astype(np.float64))
    return Workload(cfg, q16, kb, f16_bits_to_f32(q16), note="integer")


def stress60_fixture(cfg: Config, seed: int = 2060) -> Workload:
    """Literal reading of 'values up to ~60': q, k ~ U(-60, 60) rounded to fp16."""
    nq, G, H, D = cfg.nq, cfg.G, cfg.H, cfg.D
    nb_alloc = max(cfg.nb, 1)
    q = 60.0 * uniform_pm1(seed, TAG_Q, nq * G * H * D)
    k = 60.0 * uniform_pm1(seed, TAG_K, G * nb_alloc * D)
    q16 = f64_to_f16_bits(q).reshape(nq, G, H, D)
    kb = f64_to_f16_bits(k).reshape(G, nb_alloc, D)
    return Workload(cfg, q16, kb, f16_bits_to_f32(q16), note="stress60")


def conversion_fixture(cfg: Config, seed: int = 1012) -> Workload:
    """fp32 queries that are NOT fp16-exact (N(0,1)/sqrt(D) rounded to fp32
    only); the fp16 operand is whatever the conversion stage produces."""
    nq, G, H, D = cfg.nq, cfg.G, cfg.H, cfg.D
    q32 = (normal(seed, TAG_Q, nq * G * H * D) / math.sqrt(D)).astype(np.float32)
    q32 = q32.reshape(nq, G, H, D)
    nb_alloc = max(cfg.nb, 1)
    kb = f64_to_f16_bits(normal(seed, TAG_K, G * nb_alloc * D) / math.sqrt(D))
    return Workload(cfg, np.zeros((nq, G, H, D), np.uint16), kb.reshape(G, nb_alloc, D),
                    q32, note="conversion")


def fp32_bit_patterns(start: int, count: int) -> np.ndarray:
    """float32 values whose bit patterns are start, start+1, ... (< 2^32)."""
    assert 0 <= start and start + count <= 1 << 32
    return np.arange(start, start + count, dtype=np.uint64).astype(np.uint32).view(np.float32)
