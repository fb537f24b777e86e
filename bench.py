"""Benchmark of the QSA block-score select phase on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole phase over the workload's synthetic batch:
fp32 -> fp16 conversion of the queries, the MFMA full-block scorer (+ the
tail-block kernel when n_kv is not a multiple of the block size), and the
per-row top-k selector, each a C-ABI call of libqsa.so on one stream.  The
K timed steps are captured in one HIP graph (the phase at nq = 256 is a few
microseconds of GPU work, far below Python's per-call cost) and replayed once
between two events, bracketed by device synchronisation; inputs are resident
in HBM before the timed region starts.

Per-kernel durations come from graphs of K back-to-back launches of one
stage, timed with events on the same stream; the scorer's roofline uses that
duration.  The CPU baseline times the float64 oracle (never tuned) on the
host cores on the same workload.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QSA select ms + scorer TFLOP/s (fraction of FP16 MFMA peak), nq=256 @128K"
PEAK_FP16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense fp16 FLOP/clk/CU (published 2.5 PF)
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3       # dense fp32 vector (published)
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="nq256_nkv131072")
    p.add_argument("--prefill-steps", type=int, default=20,
                   help="steps for the full-prefill chunk reported beside the workload (0: skip)")
    p.add_argument("--decode-steps", type=int, default=200,
                   help="steps for the decode step reported beside the workload (0: skip)")
    p.add_argument("--sweep-steps", type=int, default=100,
                   help="steps per point of the nq = 256 context sweep, 1K-128K keys (0: skip)")
    p.add_argument("--config-steps", type=int, default=100,
                   help="steps for each of the other nq = 256 / tiny configurations (0: skip)")
    p.add_argument("--beside-steps", type=int, default=50,
                   help="launches per timing of block-key construction and attention (0: skip)")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the measured MFMA and HBM-read ceilings")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target wall time of the CPU-baseline sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy (for counter calibration)")
    p.add_argument("--fused-sweep", action="store_true",
                   help="also time the phase with and without the fused selection at 4 KV heads "
                        "x 16384 queries over 516, 1024 and 2049 blocks")
    return p.parse_args()


def _code_only(text: str) -> str:
    """C++ source without its comments and trailing blanks: what compiles."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                      # string or character literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


# The source files of each profiled kernel: the kernel and its launcher, and
# the shared header.  A stored counter figure stays valid while these are
# unchanged, whatever happens in the other kernels' files.
KERNEL_FILES = {
    "score_small": ("qsa_small.hip", "qsa_internal.h"),
    "score_full": ("qsa_score.hip", "qsa_internal.h"),
    "topk": ("qsa_topk.hip", "qsa_topk_row.h", "qsa_internal.h"),
    "score_decode": ("qsa_decode.hip", "qsa_internal.h"),
    "convert": ("qsa_convert.hip", "qsa_internal.h"),
}


def source_digest(files=None) -> str:
    """sha256 over the kernel sources' code (comments left out), to tie
    stored counter figures to the code they were taken on: the named files
    of the csrc directory, or all of them."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_block_qsa_amd", "csrc")
    for name in sorted(files if files is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """Per-launch HBM bytes from committed rocprofv3 counter summaries, valid
    only while the kernel sources are those the counters were taken on."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest(KERNEL_FILES.get(kernel)):
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def scorer_kernel(cfg):
    """The scorer kernel the phase runs for this workload (fp32 queries,
    converted on load): the decode scorer when one MFMA row block holds
    every query of a KV head (16 / head pairs), else the small scorer when
    the KV heads x groups of 64 queries number fewer than 256, else the wide
    one (head passes of up to eight heads); the tail block, when there is
    one, is scored inside the same launch.  Returns the profile key and the
    kernel's name."""
    tail = "true" if cfg.n_kv % cfg.bs else "false"
    np_ = 1 if cfg.H <= 2 else 2 if cfg.H <= 4 else 4 if cfg.H <= 8 else 8
    if cfg.nf > 0 and cfg.nq <= 16 // np_:
        return "score_decode", f"score_decode_kernel<{cfg.D},{np_},true>"
    if cfg.G * -(-cfg.nq // 64) < 256:
        # block segments give about 256 workgroups, at least one tile each;
        # fp32 queries are staged in LDS when the rows fill a workgroup's four
        # query groups, and then eight waves serve segments of two or more
        # tiles; K tiles per staged chunk and wave half: with eight waves 2
        # when a segment is a whole number of 4-tile chunks, with four 2 when
        # it holds an even number of at least four tiles
        n_tiles = -(-cfg.nf // 32)
        base = cfg.G * -(-(-(-cfg.nq // (16 // np_))) // 4)
        segs = min(-(-256 // base) if base < 256 else 1, max(n_tiles, 1))
        tps = -(-n_tiles // segs) if n_tiles else 0
        rows_fill = cfg.nq >= 4 * (16 // np_)
        nw = 8 if rows_fill and tps >= 2 else 4
        if nw == 8:
            ch = 2 if tps % 4 == 0 else 1
        else:
            ch = 2 if tps >= 4 and tps % 2 == 0 else 1
        stage = "true" if rows_fill else "false"
        return "score_small", f"score_small_kernel<{cfg.D},{np_},true,{ch},{stage},{nw}>"
    np_ = min(4, (cfg.H + 1) // 2)
    return "score_full", f"score_full_kernel<{cfg.D},{np_},false,true,{tail},true,0,false,true>"


class Phase:
    """Device buffers and raw C-ABI calls of one workload (no Python checks
    inside the hot loop: arguments are validated once by a checked call).

    The phase runs as a caller would run it: fp32 queries in, no fp16 copy
    kept, so it is two launches, the scorer (converting the queries as it
    loads them) and the selector.  Each is also timed alone: the scorer as
    the phase with k = 0 (exactly the phase's scorer launch), the selector as
    qsa_select_topk on the phase's scores.  The stand-alone conversion and
    the fp16-input scorer (qsa_block_scores) are timed for reference; they
    are not part of the phase."""

    def __init__(self, cfg, qsa, torch, w):
        import numpy as np
        self.cfg, self.qsa, self.torch = cfg, qsa, torch
        dev = torch.device("cuda:0")
        self.q32 = torch.from_numpy(w.q32).to(dev)
        self.kb = torch.from_numpy(w.kblk.view(np.float16)).to(dev)
        self.ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev)
        self.q16 = torch.empty(self.q32.shape, dtype=torch.float16, device=dev)
        self.n_q = self.q32.numel()
        L = qsa.lib
        P = qsa._ptr
        c = cfg
        ws = self.ws
        qts = c.G * c.H * c.D
        # checked once through the binding
        qsa.select_phase(self.q32, self.kb, c.n_kv, c.bs, c.k, ws)
        qsa.convert_f32_f16(self.q32, out=self.q16)
        torch.cuda.synchronize()
        self._conv = (L.qsa_convert_f32_f16, (P(self.q32), P(self.q16), self.n_q))
        self._score16 = (L.qsa_block_scores, (P(self.q16), qts, P(self.kb), self.kb.stride(0),
                                              P(ws.scores), ws.ld_s, c.G, c.nq, c.H, c.D,
                                              c.n_kv, c.bs, 0))
        self._topk = (L.qsa_select_topk, (P(ws.scores), ws.ld_s, c.rows, c.nb, c.k, P(ws.ids),
                                          c.k, None))
        phase = (P(self.q32), None, qts, P(self.kb), self.kb.stride(0), P(ws.scores), ws.ld_s,
                 P(ws.ids), c.k, None, c.G, c.nq, c.H, c.D, c.n_kv, c.bs)
        self._phase = (L.qsa_select_phase, phase + (c.k, 0, 0))
        self._score = (L.qsa_select_phase, phase + (0, 0, 0))   # k = 0: the scorer launch only
        # the phase with the selection inside the scorer's launch where the
        # fused scorer serves the shape (QSA_FUSED_SELECT = 2)
        self._phase_fused = (L.qsa_select_phase, phase + (c.k, 0, qsa.FUSED_SELECT))
        # the phase with the streaming selection where it serves the shape
        # (QSA_STREAM_SELECT = 4): no score written
        self._phase_stream = (L.qsa_select_phase, phase + (c.k, 0, qsa.STREAM_SELECT))

    def _call(self, fa):
        fn, args = fa
        st = fn(*args, self.qsa._stream(None))
        if st != 0:
            raise RuntimeError(f"{fn.__name__}: {self.qsa.status_string(st)}")

    def convert(self):
        self._call(self._conv)

    def score(self):
        self._call(self._score)

    def score16(self):
        self._call(self._score16)

    def topk(self):
        self._call(self._topk)

    def step(self):
        self._call(self._phase)

    def step_fused(self):
        self._call(self._phase_fused)

    def step_stream(self):
        self._call(self._phase_stream)


def graph_of(torch, fn, n):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    return g


def time_graph(torch, g, n) -> float:
    """ms per step of one replay of a graph holding n steps."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def median_of_9(torch, fn) -> float:
    """The pages' protocol: 3 untimed calls, then the median of 9 single
    calls, each bracketed by events and waited for (ms).  Each call carries
    its own launch cost and the idle time around it, which a graph of
    back-to-back steps hides."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(9):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return sorted(ts)[4]


def burst_median(torch, fn, reps=15, burst=5) -> float:
    """Short bursts: 2 untimed calls, then `burst` back-to-back calls between
    two events, repeated `reps` times; the median per-call time (ms).  The
    chip stays below the heat of a long graph, which the graph figures and
    the single launches do not show."""
    ts = []
    for _ in range(reps):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(burst):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / burst)
    return sorted(ts)[len(ts) // 2]


def single_call_stats(torch, fn, n=100) -> dict:
    """n single calls, each bracketed by events and waited for: median and
    the 10th and 90th percentiles (ms)."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    return {"n": n, "p10": ts[n // 10], "median": ts[n // 2], "p90": ts[(9 * n) // 10]}


class PowerClock:
    """Samples the GPU's graphics clock, socket power and hotspot temperature
    through amdsmi every ~10 ms while a measured loop runs (best effort:
    None where the library or the metric is not available)."""

    def __init__(self):
        self.ok = False
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.h = amdsmi.amdsmi_get_processor_handles()[0]
            self.amdsmi = amdsmi
            self.ok = self._read() is not None
        except Exception:   # no amdsmi, no device, no permission
            self.ok = False

    def _read(self):
        try:
            m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        except Exception:
            return None

        def num(key):
            v = m.get(key)
            return float(v) if isinstance(v, (int, float)) and v not in (0xFFFF, 0xFFFFFFFF) else None

        clk = num("current_gfxclk")
        if clk is None:
            gfx = m.get("current_gfxclks")
            if isinstance(gfx, list):
                vals = [float(x) for x in gfx if isinstance(x, (int, float)) and x not in (0xFFFF,)]
                clk = sum(vals) / len(vals) if vals else None
        return {"gfxclk_mhz": clk, "power_w": num("current_socket_power"),
                "hotspot_c": num("temperature_hotspot")}

    def sample_while(self, torch, fn, seconds: float):
        """Runs fn repeatedly for about `seconds`, sampling on a side thread."""
        import threading
        if not self.ok:
            return None
        samples, stop = [], threading.Event()

        def poll():
            while not stop.is_set():
                r = self._read()
                if r is not None:
                    samples.append(r)
                time.sleep(0.01)

        th = threading.Thread(target=poll, daemon=True)
        th.start()
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        out = {"samples": len(samples), "seconds": seconds}
        for key in ("gfxclk_mhz", "power_w", "hotspot_c"):
            v = [x[key] for x in samples if x[key] is not None]
            out[key] = ({"mean": sum(v) / len(v), "min": min(v), "max": max(v)} if v else None)
        return out


def measured_peaks(torch, power=None) -> dict | None:
    """Measured ceilings from libqsa_bench.so: the sustained rate of the
    scorers' two MFMA instructions on register-resident random fp16 operands
    (and on zeros), the better of the two being the ceiling, and the
    streaming read bandwidth of a 2 GiB buffer."""
    import ctypes
    import numpy as np
    path = os.path.join(ROOT, "sparse_attention_block_qsa_amd", "libqsa_bench.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.qsa_bench_mfma_f16.argtypes = [vp, i64, vp, c_int, c_int, c_int, vp]
    L.qsa_bench_mfma_f16_16x16x32.argtypes = [vp, i64, vp, c_int, c_int, c_int, vp]
    L.qsa_bench_read.argtypes = [vp, i64, vp, c_int, vp]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(2024)
    rand = torch.from_numpy(
        (rng.standard_normal(4096 * 8) / np.sqrt(128)).astype(np.float16)).to(dev)
    zero = torch.zeros(4096 * 8, dtype=torch.float16, device=dev)
    res = {"mfma_kernel": "v_mfma_f32_32x32x16_f16 and v_mfma_f32_16x16x32_f16 loops, operands "
                          "in registers, four (eight) accumulator chains per wave; 2 and 4 waves "
                          "per SIMD, runs of ~5 ms after a warm-up run; the best of the runs.  "
                          "'random': four A and four B fragments of N(0,1)/sqrt(128) fp16 in turn "
                          "(the scorer's operands change as often); 'random_held': one A and one "
                          "B fragment per wave; 'zero': zero operands",
           "mfma_runs": {}}
    shapes = {"32x32x16": (L.qsa_bench_mfma_f16, 2 * 32 * 32 * 16, 12000),
              "16x16x32": (L.qsa_bench_mfma_f16_16x16x32, 2 * 16 * 16 * 32, 24000)}

    def mfma_run(fn, buf, grid, iters, held, out):
        rc = fn(ctypes.c_void_p(buf.data_ptr()), buf.numel() // 8,
                ctypes.c_void_p(out.data_ptr()), grid, iters, held,
                ctypes.c_void_p(stream.cuda_stream))
        assert rc == 0, rc

    for name, buf, held in (("random", rand, 0), ("random_held", rand, 1), ("zero", zero, 0)):
        best = 0.0
        for shape, (fn, flop_per_mfma, iters0) in shapes.items():
            best_shape = 0.0
            for waves in (2, 4):
                grid = 256 * waves
                iters = iters0 // waves
                out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
                flop = grid * 4 * iters * L.qsa_bench_mfma_per_iter() * flop_per_mfma
                ts = []
                for _ in range(4):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    mfma_run(fn, buf, grid, iters, held, out)
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1))
                ts = sorted(ts[1:])
                rate = flop / (ts[len(ts) // 2] * 1e-3) / 1e12
                run = {"tflops": rate, "ms": ts[len(ts) // 2]}
                if power is not None and power.ok and waves == 2:
                    run["power_clock"] = power.sample_while(
                        torch, lambda: mfma_run(fn, buf, grid, iters, held, out), 0.4)
                res["mfma_runs"][f"{name}_{shape}_{waves}waves_per_simd"] = run
                best_shape = max(best_shape, rate)
            res[f"mfma_f16_{name}_{shape}_tflops"] = best_shape
            best = max(best, best_shape)
        res[f"mfma_f16_{name}_tflops"] = best
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    rgrid = 2048
    rout = torch.empty(rgrid * 256, dtype=torch.int32, device=dev)
    ts = []
    for _ in range(6):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = L.qsa_bench_read(ctypes.c_void_p(src.data_ptr()), nbytes // 16,
                              ctypes.c_void_p(rout.data_ptr()), rgrid,
                              ctypes.c_void_p(stream.cuda_stream))
        e1.record()
        torch.cuda.synchronize()
        assert rc == 0, rc
        ts.append(e0.elapsed_time(e1))
    ts = sorted(ts[1:])
    res["hbm_read_gbs"] = nbytes / (ts[len(ts) // 2] * 1e-3) / 1e9
    res["hbm_read_bytes"] = nbytes
    del src
    # the fixed cost of a launch: an empty kernel, timed like the stages (a
    # graph of back-to-back launches), with one workgroup and with the decode
    # scorer's grid (8 KV heads x 65 single-wave workgroups)
    L.qsa_bench_empty.argtypes = [c_int, c_int, vp]
    res["empty_launch_us"] = {}
    for grid, block in ((1, 64), (520, 64), (1024, 256)):
        fn = lambda: L.qsa_bench_empty(grid, block, ctypes.c_void_p(
            torch.cuda.current_stream().cuda_stream))
        res["empty_launch_us"][f"grid{grid}x{block}"] = _time_launches(torch, fn, 200) * 1e3
    return res


def measure(cfg, qsa, torch, steps, warmup, w=None, calls_100=False):
    import qsa_inputs as qi
    if w is None:
        w = qi.make(cfg)
    ph = Phase(cfg, qsa, torch, w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            ph.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager_ids = ph.ws.ids.clone()
    eager_scores = ph.ws.scores.clone()

    g_phase = graph_of(torch, ph.step, steps)
    # ---- timed region: exactly `steps` phase steps ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = time_graph(torch, g_phase, steps)
    wall = time.perf_counter() - t0
    # the replayed graph must reproduce the eager result bit for bit
    same = bool(torch.equal(eager_ids, ph.ws.ids) and
                torch.equal(eager_scores.view(torch.int32), ph.ws.scores.view(torch.int32)))
    del g_phase

    stages, alone = {}, {}
    for d, name, fn in ((stages, "scorer", ph.score), (stages, "topk", ph.topk),
                        (alone, "convert", ph.convert), (alone, "block_scores_f16", ph.score16),
                        (alone, "phase_fused_select", ph.step_fused)):
        if cfg.nb == 0 and name in ("scorer", "block_scores_f16"):
            d[name] = 0.0   # nothing to score: the call launches nothing
            continue
        g = graph_of(torch, fn, steps)
        d[name] = time_graph(torch, g, steps)
        del g
    # the fused form's results are the separate selector's, bit for bit
    fused_same = bool(torch.equal(eager_ids, ph.ws.ids))
    # and so are the streaming form's
    ph.ws.ids.fill_(-1)
    g = graph_of(torch, ph.step_stream, steps)
    alone["phase_stream_select"] = time_graph(torch, g, steps)
    del g
    stream_same = bool(torch.equal(eager_ids, ph.ws.ids))
    med9 = {name: median_of_9(torch, fn) for name, fn in
            (("phase", ph.step), ("scorer", ph.score), ("block_scores_f16", ph.score16),
             ("phase_fused_select", ph.step_fused), ("phase_stream_select", ph.step_stream))}
    c100 = ({name: single_call_stats(torch, fn) for name, fn in
             (("phase", ph.step), ("scorer", ph.score), ("block_scores_f16", ph.score16))}
            if calls_100 else None)
    flop = cfg.flop
    return {
        "phase": ph,
        "median_of_9_ms": med9,
        "single_calls_ms": c100,
        "ms_per_step": ms_step,
        "wall_s": wall,
        "graph_replay_matches_eager": same,
        "fused_select_matches": fused_same,
        "stream_select_matches": stream_same,
        "stages_ms": stages,
        "entry_points_ms": alone,
        "scorer_tflops": flop / (stages["scorer"] * 1e-3) / 1e12 if stages["scorer"] > 0 else 0.0,
        "block_scores_f16_tflops": (flop / (alone["block_scores_f16"] * 1e-3) / 1e12
                                    if alone["block_scores_f16"] > 0 else 0.0),
        "flop": flop,
    }


def fused_sweep(qsa, torch) -> dict:
    """The phase with the selection in the scorer's launch (QSA_FUSED_SELECT)
    against the two launches, at the prefill chunk's shape over the block
    counts the fused form serves: per point the median of three interleaved
    rounds, each a graph of 5 phases; the ids are compared bit for bit."""
    import numpy as np
    import qsa_inputs as qi
    dev = torch.device("cuda:0")
    out = []
    for n_kv in (33000, 65536, 131077):
        cfg = qi.Config("fused_sweep", 4, 16384, 8, 128, n_kv, 64, 64, "normal", 5)
        w = qi.make(cfg)
        q = torch.from_numpy(w.q32).to(dev)
        kb = torch.from_numpy(w.kblk.view(np.float16)).to(dev)
        ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev)
        times, ids = {False: [], True: []}, {}
        for _ in range(3):
            for fused in (False, True):
                fn = lambda: qsa.select_phase(q, kb, n_kv, cfg.bs, cfg.k, ws, fused_select=fused)
                for _ in range(2):
                    fn()
                torch.cuda.synchronize()
                ids[fused] = ws.ids.clone()
                g = graph_of(torch, fn, 5)
                times[fused].append(time_graph(torch, g, 5))
                del g
        out.append({"n_kv": n_kv, "nb": cfg.nb, "two_launches_us": sorted(times[False])[1] * 1e3,
                    "fused_us": sorted(times[True])[1] * 1e3,
                    "same_ids": bool(torch.equal(ids[False], ids[True]))})
        print(f"# fused sweep nb {cfg.nb}: two launches {out[-1]['two_launches_us']:.1f} us, "
              f"fused {out[-1]['fused_us']:.1f} us, same ids {out[-1]['same_ids']}",
              file=sys.stderr, flush=True)
        del q, kb, ws, w
    return {"workload": "4 KV heads x 16384 queries, H 8, D 128, bs 64, k 64", "points": out}


def _time_launches(torch, fn, n) -> float:
    """ms per launch of a graph of n back-to-back launches (after 3 eager)."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    g = graph_of(torch, fn, n)
    ms = time_graph(torch, g, n)
    del g
    return ms


def measure_beside(qsa, torch, n, peaks) -> dict:
    """The block keys of the full-prefill chunk built from token keys
    (HBM-bound: 2*D bytes per token and KV head read, 2*D per block written)
    and attention over the selection phase's ids at nq = 256 with 128K keys
    and at the decode step (per row k*bs tokens gathered: 4*D bytes of keys
    and values per token and KV head; 4*D FLOP per token and query head)."""
    import numpy as np
    import qsa_inputs as qi
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(9)
    out = {}
    pc = qi.PREFILL
    kt = torch.from_numpy(qi.f64_to_f16_bits(rng.standard_normal((pc.n_kv, pc.G, pc.D))
                                             / np.sqrt(pc.D)).view(np.float16)).to(dev)
    kb = torch.empty((pc.G, pc.nb, pc.D), dtype=torch.float16, device=dev)
    qsa.block_keys(kt, pc.n_kv, pc.bs, out=kb)
    L = qsa.lib
    args = (qsa._ptr(kt), kt.stride(0), qsa._ptr(kb), kb.stride(0), pc.G, pc.D, pc.n_kv, pc.bs)
    ms = _time_launches(torch, lambda: L.qsa_block_keys(*args, qsa._stream(None)), n)
    nbytes = 2.0 * pc.D * pc.G * (pc.n_kv + pc.nb)
    out["block_keys"] = {"workload": pc.name, "us": ms * 1e3, "bytes": nbytes,
                         "gbs": nbytes / (ms * 1e-3) / 1e9,
                         "frac_of_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "frac_of_measured_read": (nbytes / (ms * 1e-3) / 1e9 / peaks["hbm_read_gbs"]
                                                   if peaks else None)}
    del kt, kb
    out["attention"] = {}
    for cfg in (qi.HEADLINE, qi.DECODE):
        w = qi.make(cfg)
        q16 = torch.from_numpy(w.q16.view(np.float16)).to(dev)
        kv = [torch.from_numpy(qi.f64_to_f16_bits(rng.standard_normal((cfg.n_kv, cfg.G, cfg.D)))
                               .view(np.float16)).to(dev) for _ in range(2)]
        ws = qsa.PhaseWorkspace(cfg.nq, cfg.G, cfg.H, cfg.D, cfg.n_kv, cfg.bs, cfg.k, dev)
        ids = qsa.select_phase(torch.from_numpy(w.q32).to(dev),
                               torch.from_numpy(w.kblk.view(np.float16)).to(dev), cfg.n_kv, cfg.bs,
                               cfg.k, ws)
        o = qsa.sparse_attention(q16, kv[0], kv[1], ids, cfg.n_kv, cfg.bs, ws=None)
        aws = qsa.attention_workspace(cfg.G, cfg.nq, cfg.H, cfg.D, cfg.bs, cfg.k, dev)
        torch.cuda.synchronize()
        ids_np = ids.cpu().numpy()
        nb = cfg.nb
        toks = sum(min(cfg.bs, cfg.n_kv - int(b) * cfg.bs) for b in ids_np.ravel() if 0 <= b < nb)
        a = (qsa._ptr(q16), cfg.G * cfg.H * cfg.D, qsa._ptr(kv[0]), qsa._ptr(kv[1]), cfg.G * cfg.D,
             qsa._ptr(ids), cfg.k, qsa._ptr(o), cfg.G * cfg.H * cfg.D, cfg.G, cfg.nq, cfg.H, cfg.D,
             cfg.n_kv, cfg.bs, cfg.k, qsa._ptr(aws), 0 if aws is None else aws.numel())
        ms = _time_launches(torch, lambda: L.qsa_sparse_attention(*a, qsa._stream(None)), n)
        flop = 4.0 * toks * cfg.H * cfg.D
        gathered = 4.0 * toks * cfg.D
        out["attention"][cfg.name] = {
            "us": ms * 1e3, "tokens_attended": toks, "flop": flop,
            "tflops": flop / (ms * 1e-3) / 1e12,
            "frac_of_fp32_vector_peak": flop / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
            "gathered_bytes": gathered, "gathered_gbs": gathered / (ms * 1e-3) / 1e9,
            "workgroups_per_row": (aws.numel() // (cfg.rows * cfg.H * (2 + cfg.D))
                                   if aws is not None else 1)}
        del q16, kv, ws, ids, o, aws
    return out


def config_summary(cfg, r) -> dict:
    """One workload reported the way the headline is."""
    st, al = r["stages_ms"], r["entry_points_ms"]
    return {"G": cfg.G, "nq": cfg.nq, "H": cfg.H, "D": cfg.D, "n_kv": cfg.n_kv, "bs": cfg.bs,
            "nb": cfg.nb, "k": cfg.k, "flop": cfg.flop,
            "select_ms": r["ms_per_step"], "scorer_ms": st["scorer"], "topk_ms": st["topk"],
            "scorer_tflops": r["scorer_tflops"],
            "scorer_frac_of_peak": r["scorer_tflops"] / PEAK_FP16_TFLOPS,
            "block_scores_f16_ms": al["block_scores_f16"],
            "block_scores_f16_tflops": r["block_scores_f16_tflops"],
            "convert_ms": al["convert"],
            "median_of_9_ms": r["median_of_9_ms"],
            "graph_replay_matches_eager": r["graph_replay_matches_eager"]}


def _oracle_time(w, cfg, target_s, max_reps=1000) -> tuple[float, int, float, float, float]:
    """Seconds per whole-workload oracle pass (scores + S + B, then top-k),
    repeated until about target_s of wall time; also the two stages' seconds
    per pass (fixture generation excluded)."""
    import oracle
    reps, t_scores, t_topk = 0, 0.0, 0.0
    while True:
        t0 = time.perf_counter()
        ref = oracle.scores(w.q16, w.kblk, cfg.nb)
        t1 = time.perf_counter()
        oracle.topk(ref.score, cfg.k)
        t2 = time.perf_counter()
        t_scores += t1 - t0
        t_topk += t2 - t1
        reps += 1
        if t_scores + t_topk >= target_s or reps >= max_reps:
            break
    tot = t_scores + t_topk
    return tot / reps, reps, tot, t_scores / reps, t_topk / reps


def cpu_model() -> str | None:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, target_s, single_thread_cfgs=()):
    """The float64 oracle (scores + S + B, then top-k), as it stands, on the
    host cores: whole workload, repeated until about target_s of wall time;
    then one thread on each of single_thread_cfgs."""
    import oracle
    import qsa_inputs as qi
    w = qi.make(cfg)
    per, reps, tot, per_scores, per_topk = _oracle_time(w, cfg, target_s)
    threads = oracle.max_threads()
    single = {}
    if single_thread_cfgs:
        oracle.set_threads(1)
        try:
            for c in single_thread_cfgs:
                wc = qi.make(c)
                p1, n1, _, s1, k1 = _oracle_time(wc, c, 0.5, max_reps=20)
                single[c.name] = {"ms": p1 * 1e3, "scores_ms": s1 * 1e3, "topk_ms": k1 * 1e3,
                                  "tflops": c.flop / p1 / 1e12, "reps": n1}
        finally:
            oracle.set_threads(threads)
    return {"value": cfg.flop / per / 1e12, "unit": "TFLOP/s", "cores": threads,
            "cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "kind": "oracle", "ms_per_step": per * 1e3,
            "scores_ms": per_scores * 1e3, "topk_ms": per_topk * 1e3,
            "sample": f"whole {cfg.name} workload ({cfg.rows} rows x {cfg.nb} blocks: scores, "
                      f"S, B in float64 and top-{cfg.k}), {reps} repetition(s), {tot:.1f} s, "
                      f"{threads} OpenMP threads",
            "single_thread": single}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the select phase is per-GPU work with no collective (each GPU runs it over the "
              "KV heads or the block range it holds)", file=sys.stderr)
        sys.exit(2)
    import torch

    import qsa_inputs as qi
    import sparse_attention_block_qsa_amd as qsa

    cfg = qi.CONFIGS[args.workload]
    print(f"# workload {cfg.name}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
          flush=True)
    res = measure(cfg, qsa, torch, args.steps, args.warmup, calls_100=True)
    print(f"# {cfg.name}: {res['ms_per_step'] * 1e3:.2f} us/step, stages "
          f"{ {k: round(v * 1e3, 2) for k, v in res['stages_ms'].items()} } us, alone "
          f"{ {k: round(v * 1e3, 2) for k, v in res['entry_points_ms'].items()} } us",
          file=sys.stderr, flush=True)

    scorer_ms = res["stages_ms"]["scorer"]
    achieved = res["flop"] / (scorer_ms * 1e-3) / 1e12
    kernel, kernel_desc = scorer_kernel(cfg)

    power = PowerClock()
    peaks = measured_peaks(torch, power) if not args.no_peaks else None
    if peaks:
        print(f"# measured: mfma f16 {peaks['mfma_f16_random_tflops']:.0f} TFLOP/s random operands, "
              f"{peaks['mfma_f16_zero_tflops']:.0f} zeros; HBM read {peaks['hbm_read_gbs']:.0f} GB/s; "
              f"empty launch {peaks['empty_launch_us']} us", file=sys.stderr, flush=True)
    roofline = {"bound": "mfma", "kernel": kernel_desc,
                "achieved": achieved, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_FP16_TFLOPS,
                "traffic": read_traffic(kernel, cfg.name),
                "per_launch_flop": res["flop"], "launch_ms": scorer_ms,
                "measured_peak": peaks["mfma_f16_random_tflops"] if peaks else None,
                "frac_of_measured_peak": achieved / peaks["mfma_f16_random_tflops"] if peaks else None}
    power_clock = {"headline_phase": power.sample_while(torch, res["phase"].step, 0.3)} \
        if power.ok else None

    # the other configurations, reported the same way (Tiny with n_kv = 0 too)
    configs = {}
    if args.config_steps > 0:
        for name in ("tiny_nq37_nkv1000", "nq256_nkv4096", "nq256_nkv32768"):
            if name == cfg.name:
                continue
            c = qi.CONFIGS[name]
            r = measure(c, qsa, torch, args.config_steps, 10)
            configs[name] = config_summary(c, r)
            print(f"# {name}: phase {r['ms_per_step'] * 1e3:.2f} us, scorer "
                  f"{r['stages_ms']['scorer'] * 1e3:.2f} us, topk {r['stages_ms']['topk'] * 1e3:.2f} us",
                  file=sys.stderr, flush=True)
            del r
        w0 = qi.make(qi.TINY, n_kv=0)   # the empty case: no scores, every id -1
        r = measure(w0.cfg, qsa, torch, args.config_steps, 10, w=w0)
        configs["tiny_nq37_nkv0"] = config_summary(w0.cfg, r)
        del r

    prefill = None
    if args.prefill_steps > 0 and cfg.name != qi.PREFILL.name:
        pc = qi.PREFILL
        print(f"# prefill chunk {pc.name}: steps {args.prefill_steps}", file=sys.stderr,
              flush=True)
        pr = measure(pc, qsa, torch, args.prefill_steps, 3)
        if power.ok:
            power_clock["prefill_phase"] = power.sample_while(torch, pr["phase"].step, 0.5)
            power_clock["prefill_scorer_f16"] = power.sample_while(torch, pr["phase"].score16, 0.5)
        ps = pr["stages_ms"]
        burst = {"scorer": burst_median(torch, pr["phase"].score),
                 "block_scores_f16": burst_median(torch, pr["phase"].score16)}
        hbm = {"convert": 6.0 * pc.nq * pc.G * pc.H * pc.D,
               "topk": 4.0 * pc.rows * pc.nb + 4.0 * pc.rows * pc.k}
        pe = pr["entry_points_ms"]
        prefill = {
            "workload": pc.name, "ms_per_step": pr["ms_per_step"], "stages_ms": ps,
            "entry_points_ms": pe,
            "scorer_tflops": pr["scorer_tflops"],
            "scorer_frac_of_peak": pr["scorer_tflops"] / PEAK_FP16_TFLOPS,
            "scorer_kernel": scorer_kernel(pc)[1],
            "scorer_traffic_bytes": read_traffic(scorer_kernel(pc)[0], pc.name),
            "convert_gbs": hbm["convert"] / (pe["convert"] * 1e-3) / 1e9,
            "convert_traffic_bytes": read_traffic("convert", pc.name),
            "convert_gbs_counters": (read_traffic("convert", pc.name) / (pe["convert"] * 1e-3) / 1e9
                                     if read_traffic("convert", pc.name) else None),
            "block_scores_f16_frac_of_peak":
                pc.flop / (pe["block_scores_f16"] * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
            "topk_gbs": hbm["topk"] / (ps["topk"] * 1e-3) / 1e9,
            "topk_kernel": "topk_kernel<33,true>",
            "topk_traffic_bytes": read_traffic("topk", pc.name),
            "topk_gbs_counters": (read_traffic("topk", pc.name) / (ps["topk"] * 1e-3) / 1e9
                                  if read_traffic("topk", pc.name) else None),
            "topk_frac_of_measured_read": (hbm["topk"] / (ps["topk"] * 1e-3) / 1e9
                                           / peaks["hbm_read_gbs"] if peaks else None),
            "block_scores_f16_frac_of_measured_peak":
                (pc.flop / (pe["block_scores_f16"] * 1e-3) / 1e12 / peaks["mfma_f16_random_tflops"]
                 if peaks else None),
            "scorer_frac_of_measured_peak":
                (pr["scorer_tflops"] / peaks["mfma_f16_random_tflops"] if peaks else None),
            "graph_replay_matches_eager": pr["graph_replay_matches_eager"],
            # the phase with the selection fused into the scorer's launch
            # (QSA_FUSED_SELECT), same ids bit for bit
            "phase_fused_select_ms": pe["phase_fused_select"],
            "phase_fused_select_median_of_9_ms": pr["median_of_9_ms"]["phase_fused_select"],
            "fused_select_matches": pr["fused_select_matches"],
            # the phase with the streaming selection (QSA_STREAM_SELECT): no
            # score written, same ids bit for bit
            "phase_stream_select_ms": pe["phase_stream_select"],
            "phase_stream_select_median_of_9_ms": pr["median_of_9_ms"]["phase_stream_select"],
            "stream_select_matches": pr["stream_select_matches"],
            # single launches timed by the pages' protocol (3 warmups, median of 9)
            "median_of_9_ms": pr["median_of_9_ms"],
            "scorer_frac_of_peak_median_of_9":
                pc.flop / (pr["median_of_9_ms"]["scorer"] * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
            "block_scores_f16_frac_of_peak_median_of_9":
                pc.flop / (pr["median_of_9_ms"]["block_scores_f16"] * 1e-3) / 1e12
                / PEAK_FP16_TFLOPS,
            # bursts of 5 back-to-back launches (median over 15 bursts)
            "burst_of_5_ms": burst,
            "scorer_frac_of_peak_burst_of_5":
                pc.flop / (burst["scorer"] * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
            "block_scores_f16_frac_of_peak_burst_of_5":
                pc.flop / (burst["block_scores_f16"] * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
        }
        print(f"# prefill: {pr['ms_per_step']:.3f} ms/step, scorer {pr['scorer_tflops']:.0f} "
              f"TFLOP/s; median of 9 single launches: phase "
              f"{pr['median_of_9_ms']['phase'] * 1e3:.1f} us, scorer "
              f"{pr['median_of_9_ms']['scorer'] * 1e3:.1f} us, fp16-input scorer "
              f"{pr['median_of_9_ms']['block_scores_f16'] * 1e3:.1f} us; fused-select phase "
              f"{pe['phase_fused_select'] * 1e3:.1f} us (graph), "
              f"{pr['median_of_9_ms']['phase_fused_select'] * 1e3:.1f} us (median of 9), same ids "
              f"{pr['fused_select_matches']}; streaming-select phase "
              f"{pe['phase_stream_select'] * 1e3:.1f} us (graph), "
              f"{pr['median_of_9_ms']['phase_stream_select'] * 1e3:.1f} us (median of 9), same ids "
              f"{pr['stream_select_matches']}; bursts of 5: scorer {burst['scorer'] * 1e3:.1f} us, "
              f"fp16-input scorer {burst['block_scores_f16'] * 1e3:.1f} us", file=sys.stderr,
              flush=True)

    decode = None
    if args.decode_steps > 0 and cfg.name != qi.DECODE.name:
        dc = qi.DECODE
        print(f"# decode step {dc.name}: steps {args.decode_steps}", file=sys.stderr, flush=True)
        dr = measure(dc, qsa, torch, args.decode_steps, 20)
        ds = dr["stages_ms"]
        # the scorer streams every KV head's block keys once: HBM-bound
        # (fp32 queries read, fp32 scores written)
        kbytes = 2.0 * dc.G * dc.nb * dc.D
        sbytes = kbytes + 4.0 * dc.rows * dc.H * dc.D + 4.0 * dc.rows * dc.nb
        decode = {
            "workload": dc.name, "ms_per_step": dr["ms_per_step"], "stages_ms": ds,
            "entry_points_ms": dr["entry_points_ms"],
            "scorer_kernel": scorer_kernel(dc)[1],
            "scorer_bytes": sbytes,
            "scorer_gbs": sbytes / (ds["scorer"] * 1e-3) / 1e9,
            "scorer_frac_of_hbm": sbytes / (ds["scorer"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "scorer_traffic_bytes": read_traffic(scorer_kernel(dc)[0], dc.name),
            # an empty kernel of the scorer's grid, timed the same way: the
            # part of the scorer's time no kernel can avoid
            "empty_launch_us_same_grid": (peaks["empty_launch_us"]["grid520x64"]
                                          if peaks else None),
            "graph_replay_matches_eager": dr["graph_replay_matches_eager"],
        }
        print(f"# decode: {dr['ms_per_step'] * 1e3:.2f} us/step, scorer {ds['scorer'] * 1e3:.2f} us",
              file=sys.stderr, flush=True)

    # nq = 256 across context lengths 1K-128K keys, the headline's shape
    # otherwise (k = 64: rows shorter than 64 blocks pad with -1)
    sweep = None
    if args.sweep_steps > 0 and cfg.name == qi.HEADLINE.name:
        sweep = []
        for n_kv in (1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072):
            ws_ = qi.make(cfg, n_kv=n_kv)
            r = measure(ws_.cfg, qsa, torch, args.sweep_steps, 10, w=ws_)
            sweep.append({"n_kv": n_kv, "nb": ws_.cfg.nb, "k": ws_.cfg.k,
                          "phase_us": r["ms_per_step"] * 1e3,
                          "scorer_us": r["stages_ms"]["scorer"] * 1e3,
                          "topk_us": r["stages_ms"]["topk"] * 1e3,
                          "scorer_tflops": r["scorer_tflops"],
                          "scorer_frac_of_peak": r["scorer_tflops"] / PEAK_FP16_TFLOPS})
            print(f"# sweep n_kv {n_kv}: phase {sweep[-1]['phase_us']:.2f} us, scorer "
                  f"{sweep[-1]['scorer_us']:.2f} us, topk {sweep[-1]['topk_us']:.2f} us",
                  file=sys.stderr, flush=True)

    # the steps beside the phase: block keys built from token keys (the step
    # before) and attention over the selected blocks (the step after)
    beside = None
    if args.beside_steps > 0:
        beside = measure_beside(qsa, torch, args.beside_steps, peaks)
        print(f"# block keys {beside['block_keys']['us']:.1f} us "
              f"({beside['block_keys']['gbs']:.0f} GB/s); attention "
              + ", ".join(f"{k} {v['us']:.1f} us" for k, v in beside["attention"].items()),
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, args.cpu_seconds,
                           single_thread_cfgs=[qi.CONFIGS[n] for n in
                                               ("nq256_nkv4096", "nq256_nkv32768", "nq256_nkv131072")])

    sweep_fused = fused_sweep(qsa, torch) if args.fused_sweep else None

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    line = {
        "metric": METRIC,
        "value": achieved,
        "value_is": "scorer TFLOP/s: FLOP of every (query, block) cell / duration of the phase's "
                    "scorer launch (fp32 queries converted on load, full blocks and tail); "
                    "select_ms is the whole phase",
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded splitmix64 N(0,1)/sqrt(D), fp16 operands, fp32 accumulation)",
        "config": {"workload": cfg.name, "G": cfg.G, "nq": cfg.nq, "H": cfg.H, "D": cfg.D,
                   "n_kv": cfg.n_kv, "bs": cfg.bs, "k": cfg.k, "parallelism": "single GPU"},
        "select_ms": res["ms_per_step"],
        "scorer_ms": scorer_ms,
        "scorer_tflops": achieved,
        "scorer_frac_of_peak": achieved / PEAK_FP16_TFLOPS,
        "block_scores_f16_tflops": res["block_scores_f16_tflops"],
        "single_calls_ms": res["single_calls_ms"],
        "measured_peaks": peaks,
        "power_clock": power_clock,
        "configs": configs,
        "stages_ms": res["stages_ms"],
        "entry_points_ms": res["entry_points_ms"],
        "median_of_9_ms": res["median_of_9_ms"],
        "graph_replay_matches_eager": res["graph_replay_matches_eager"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "full_prefill": prefill,
        "decode": decode,
        "context_sweep": sweep,
        "beside_the_phase": beside,
        "fused_select_sweep": sweep_fused,
        "source_digest": source_digest(),
        "kernel_digests": {k: source_digest(f) for k, f in KERNEL_FILES.items()},
        "context": {"pages_rx7900xtx_gfx1100_scores_ms_128k": {"warp": 2.627, "wmma": 0.252},
                    "note": "other hardware; context only"},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
