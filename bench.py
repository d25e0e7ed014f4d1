"""Benchmark of the GQA hot path on one MI355X; prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R] [--only a,b]
                    [--no-cpu-baseline] [--quick]

Headline (``value``): KV-read GB/s of one GQA decode step on the Llama-7B-sized
layer (B=16, H=32 query heads, G=8 K/V heads, d=128, cache length 1024, bf16),
i.e. algorithmic bytes (K and V actually attended, plus q, out and the
lengths) divided by the time per call.  Inputs are resident in HBM; every call
reads a different replica of the cache, rotating over >= 1 GiB of replicas, so
the 256 MB last-level cache cannot serve a call from an earlier one.

Timing: K calls are captured into one HIP graph (the library launches on the
capturing stream) and the graph is replayed R times (default 7), each replay
bracketed by a device synchronisation and timed with HIP events on the launch
stream, queued behind a ~150 us read of 1 GiB so that the host's graph launch
overlaps it and the events bracket exactly the K calls; the per-call time of a replay is its elapsed time / K, and the line
reports the median (``ms_per_step``) and the minimum.  Graph replay keeps the
host's per-call dispatch cost (Python, ctypes, argument checks) out of the
measurement, so the figure is the GPU's: kernel time plus the gap between
back-to-back kernels.  After timing, the graph's output is compared bit for
bit with an eager call of the same step.  The headline is timed with exactly
K = --steps calls per replay; every other workload with enough calls for a
replay of >= 50 ms (and >= 200 calls).  Every plain decode is also timed a
second way, as K back-to-back calls of the C entry point made directly from
C behind the same 1 GiB read (``direct_call_loop_ms_per_call``, median of R
runs).  A graph replay carries a fixed ~10 us of device-side cost, so a
headline of fewer than 200 steps reports the direct calls instead (at 20
steps: 14.6 us per step against 14.8 by graph replay; at 4000: 14.5 against
14.3, the kernel trace's 14.3).

Also reported, each with its own roofline block (``secondary``): the G sweep
{32, 8, 4, 1} on the same queries with a linear fit of time against bytes
(fixed cost and marginal bandwidth), the tiny float32 decode (latency), the
T5-XXL-sized cross-attention step, the ragged 32k-context step, IEEE-half and
fused-append decode, GQKVA decode, the causal prefill (TFLOP/s against the
bf16 matrix peak), a prompt chunk after a cached prefix, the K/V mean-pool,
the single-launch cold latency of each decode/prefill step, and an own
non-temporal 128-bit HBM read probe (``hbm_read_probe``, the measured
ceiling every memory-bound figure is also given against).  The float64 oracle
is timed on the host cores on bounded samples of each workload
(``cpu_baseline``), and the GPU's errors against it are reported there.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0         # MI355X dense bf16 matrix, published
REPS = 7                          # timed graph replays per workload
MIN_REP_MS = 50.0                 # each replay of a secondary workload lasts at least this
MIN_CALLS = 200                   # ... and holds at least this many calls
MAX_CALLS = 20000
PREFILL_WARMUP = 120              # untimed prefill calls before timing (clock ramp-up)
HEADLINE = ("llama7b_decode_bf16", 8)
METRIC = "decode KV-read GB/s (% of HBM peak) + tokens/s; prefill TFLOP/s (% MFMA)"
KERNEL_SOURCE_DIR = os.path.join("grouped_query_decode_amd", "csrc")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
TRACE_FILE = os.path.join(ROOT, "profiles", "bench_kernel_trace.md")
DEV = "cuda:0"


# ---------------------------------------------------------------------------
# accounting (algorithmic bytes and flops)
# ---------------------------------------------------------------------------

def decode_bytes(B, H, G, d, total_positions, itemsize):
    """K and V rows actually attended, plus q, out and the lengths."""
    return 2 * G * total_positions * d * itemsize + 2 * B * H * d * itemsize + 4 * B


def decode_flops(H, total_positions, d):
    return 4 * H * total_positions * d


def prefill_flops(B, T, H, d):
    return 2 * B * H * d * T * (T + 1)


def split_partial_bytes(B, H, d, S):
    """Split-N partials written once and read back once (overhead, not algorithmic)."""
    return 0 if S <= 1 else 2 * B * H * S * (d + 2) * 4


def kernel_source_hash():
    """Hash of every library source (kernels, host side, headers)."""
    h = hashlib.sha256()
    base = os.path.join(ROOT, KERNEL_SOURCE_DIR)
    files = sorted(f for f in os.listdir(base) if f.endswith((".hip", ".cpp", ".h")))
    for f in files + [os.path.join("..", "..", "include", "gqa.h")]:
        with open(os.path.join(base, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _stored_json(path):
    """The JSON block of a committed profile summary, if it was taken from these sources."""
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), flags=re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    return data if data.get("kernel_source_sha256_16") == kernel_source_hash() else None


def stored_traffic():
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) per workload, from the committed
    counter summary, while it still matches the library sources."""
    data = _stored_json(COUNTERS_FILE)
    return {} if data is None else data.get("traffic_bytes_per_launch", {})


def stored_kernel_means():
    """rocprofv3 mean kernel duration (us) per workload from the committed trace summary."""
    data = _stored_json(TRACE_FILE)
    return {} if data is None else data.get("kernel_mean_us", {})


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def _eager_ms(torch, fn, n_calls):
    """Rough per-call time of back-to-back eager calls (used only to size the graphs)."""
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n_calls):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n_calls


def calls_for(ms_per_call, min_rep_ms=None):
    """Calls per timed replay: at least MIN_CALLS and at least min_rep_ms of work."""
    rep_ms = MIN_REP_MS if min_rep_ms is None else min_rep_ms
    return int(min(MAX_CALLS, max(MIN_CALLS, math.ceil(rep_ms / max(ms_per_call, 1e-6)))))


# Device work queued ahead of each timed replay (set once the cache-evicting
# read exists): a ~150 us read of 1 GiB, during which the host submits the
# graph, so the start event is taken when the first timed kernel can start
# and a replay of a few calls does not carry the graph launch's host latency
# (~9 us: 20 calls of the headline step read 14.8 us per call without it,
# 14.3 with it and with 4000 calls).
LEAD = None


def graph_time(torch, fn, n_calls, warmup, reps=REPS, out=None):
    """Per-call milliseconds of fn(0) .. fn(n_calls-1) captured into one HIP graph.

    ``warmup`` eager calls first; then one untimed replay and ``reps`` timed
    replays, each bracketed by torch.cuda.synchronize() and timed with events
    on the launch stream (behind LEAD's read, when set, so that the events
    bracket exactly the calls).  With ``out`` (the tensor the calls write), the
    graph result is compared bit for bit with an eager repeat of the last call.
    """
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n_calls):
            fn(i)
    stream = torch.cuda.current_stream()
    graph.replay()
    torch.cuda.synchronize()
    per_call = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        if LEAD is not None:
            LEAD()
        a.record(stream)
        graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per_call.append(a.elapsed_time(b) / n_calls)
    same = None
    if out is not None:
        from_graph = out.clone()
        fn(n_calls - 1)
        torch.cuda.synchronize()
        same = bool(torch.equal(from_graph.view(torch.uint8), out.view(torch.uint8)))
    del graph
    return {"median_ms": statistics.median(per_call), "min_ms": min(per_call),
            "rep_ms": [round(x, 6) for x in per_call], "calls_per_rep": n_calls,
            "graph_matches_eager": same}


class ColdFlusher:
    """A single timed launch from cold caches: queued right behind a read of 1 GiB
    (which evicts the last-level cache and lasts ~150 us, longer than the host
    takes to enqueue the events and the call), so the events bracket the
    launch's device time and no host dispatch time."""

    def __init__(self, torch, probe):
        self.torch = torch
        self.probe = probe
        self.buf = torch.ones(1 << 30, dtype=torch.uint8, device=DEV)

    def lead(self):
        """Enqueue the 1 GiB read (no host wait): device work ahead of a timed region."""
        self.probe.read(self.buf, blocks=2048, unroll=8)

    def latency_us(self, fn, i):
        torch = self.torch
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        self.probe.read(self.buf, blocks=2048, unroll=8)
        a.record(stream)
        fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return round(a.elapsed_time(b) * 1e3, 2)


class ReadProbe:
    """ctypes binding of libgqa_probe.so (the benchmark's own HBM read probe)."""

    def __init__(self, torch):
        import grouped_query_decode_amd as gqa
        path = os.path.join(os.path.dirname(gqa.library_path()), "libgqa_probe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        self.lib = ctypes.CDLL(path)
        self.lib.gqa_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        self.lib.gqa_probe_hbm_read.restype = ctypes.c_int
        self.torch = torch
        self.sink = torch.zeros(4, dtype=torch.int32, device=DEV)

    def valu_rates(self, blocks=1024):
        """SIMD cycles per wave64 instruction (fma, exp, and a 1:1 mix), at the measured clock."""
        torch = self.torch
        lib = self.lib
        lib.gqa_probe_valu_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.gqa_probe_valu_rate.restype = ctypes.c_int
        out = torch.empty(blocks * 256, dtype=torch.float32, device=DEV)
        stream = torch.cuda.current_stream()
        res = {}
        for kind, name, per_step in ((0, "fma", 8), (1, "exp", 8), (2, "exp_plus_fma", 16)):
            call = lambda: lib.gqa_probe_valu_rate(ctypes.c_void_p(out.data_ptr()), kind, blocks,  # noqa: E731
                                                   ctypes.c_void_p(stream.cuda_stream))
            call()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(5):
                call()
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / 5
            # wave-instructions per SIMD: blocks x 4 waves / 1024 SIMDs x 4096 steps x per_step
            wi = blocks * 4 / 1024 * 4096 * per_step
            res[name] = {"ns_per_wave_instruction_per_simd": round(ms * 1e6 / wi, 4)}
        return res

    def lds_rates(self, blocks=512):
        """LDS cycles per wave instruction per compute unit (ds_read_b128, and ds_read_b64_tr_b16 at
        the causal prefill's V^T addresses), at the clock the chip reports for the run."""
        torch = self.torch
        lib = self.lib
        lib.gqa_probe_lds_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.gqa_probe_lds_rate.restype = ctypes.c_int
        stream = torch.cuda.current_stream()
        res = {}
        for kind, name, lane_bytes in ((0, "ds_read_b128", 16), (1, "ds_read_b64_tr_b16_prefill_vt", 8)):
            call = lambda: lib.gqa_probe_lds_rate(ctypes.c_void_p(self.sink.data_ptr()), kind, blocks,  # noqa: E731
                                                  ctypes.c_void_p(stream.cuda_stream))
            if call() != 0:
                raise RuntimeError("gqa_probe_lds_rate refused its launch")
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(5):
                call()
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / 5
            # wave-instructions per CU: blocks x 4 waves / 256 CUs x 4096 steps x 8
            wi = blocks * 4 / 256 * 4096 * 8
            res[name] = {"ns_per_wave_instruction_per_cu": round(ms * 1e6 / wi, 4),
                         "bytes_per_ns_per_cu": round(64 * lane_bytes * wi / (ms * 1e6), 1)}
        return res

    def decode_call_loop(self, gqa, xs, out, ws, B, H, G, d, N, scale, n_calls, warmup=20, reps=3,
                         lead=None):
        """Per-call ms of n_calls back-to-back gqa_decode_split calls made directly from C
        (gqa_probe_time_decode_calls; no Python, no graph), rotating over the input sets
        xs, ``reps`` runs -- each queued behind a read of ``lead`` (a device buffer) when
        given.  Returns the per-run figures."""
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        f = self.lib.gqa_probe_time_decode_calls
        f.argtypes = ([vp] * 5 + [i32, vp] + [i32] * 5 + [ctypes.c_float] + [i32] * 2 +
                      [vp, ctypes.c_size_t, i32, i32, vp, ctypes.c_size_t, vp, vp, vp])
        f.restype = i32
        lead_ptr = vp(0) if lead is None else vp(lead.data_ptr())
        lead_bytes = 0 if lead is None else lead.numel() * lead.element_size()
        R = len(xs)
        arr = lambda key: (vp * R)(*[x[key].data_ptr() for x in xs])  # noqa: E731
        q, k, v, sl = arr("q"), arr("k_cache"), arr("v_cache"), arr("seqlens")
        fn = ctypes.cast(gqa.load_library().gqa_decode_split, vp)
        stream = vp(self.torch.cuda.current_stream().cuda_stream)
        runs = []
        for _ in range(reps):
            ms = ctypes.c_float(0.0)
            rc = f(fn, q, k, v, sl, R, vp(out.data_ptr()), B, H, G, d, N, scale, gqa.DTYPE_CODES[out.dtype], 0,
                   vp(ws.data_ptr()), ws.numel() * ws.element_size(), warmup, n_calls, lead_ptr, lead_bytes,
                   vp(self.sink.data_ptr()), stream, ctypes.byref(ms))
            if rc != 0:
                raise RuntimeError(f"gqa_probe_time_decode_calls failed ({rc})")
            runs.append(ms.value / n_calls)
        return runs

    def read(self, buf, blocks, unroll):
        rc = self.lib.gqa_probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                         ctypes.c_void_p(self.sink.data_ptr()), blocks, unroll,
                                         ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"gqa_probe_hbm_read failed ({rc})")


def bench_read_probe(torch, probe, reps):
    """Own 128-bit non-temporal read probe over 2 GiB (8x the last-level cache):
    the best of a few launch shapes is the measured read ceiling."""
    buf = torch.ones(1 << 31, dtype=torch.uint8, device=DEV)
    shapes = {}
    for blocks, unroll in ((1024, 8), (2048, 8), (2048, 16), (4096, 8), (4096, 16)):
        t = graph_time(torch, lambda i: probe.read(buf, blocks, unroll), 160, 3, reps=reps)
        shapes[f"{blocks}x256_u{unroll}"] = round(buf.numel() / (t["median_ms"] * 1e-3) / 1e9, 1)
    best = max(shapes, key=shapes.get)
    del buf
    torch.cuda.empty_cache()
    return {"bytes_per_call": 1 << 31, "GBps": shapes[best], "best_shape": best, "shapes_GBps": shapes,
            "frac_hbm_peak": round(shapes[best] / HBM_PEAK_GBPS, 4)}


def probe_at_size(torch, probe, nbytes, reps, cache):
    """The read probe over exactly ``nbytes`` per call (windows rotating over
    2 GiB, so no call is served by the last-level cache), best of a few launch
    shapes: the read rate a streaming kernel reaches at this transfer size,
    fixed launch and latency costs included."""
    key = int(nbytes)
    if key in cache:
        return cache[key]
    if "buf" not in cache:
        cache["buf"] = torch.ones(1 << 31, dtype=torch.uint8, device=DEV)
    buf = cache["buf"]
    # (transfers beyond the 2 GiB buffer: its whole size, where the rate no longer depends on size)
    n = max(16, (min(int(nbytes), buf.numel()) // 16) * 16)
    nwin = max(1, buf.numel() // n)
    views = [buf[i * n:(i + 1) * n] for i in range(nwin)]
    best = None
    for blocks, unroll in ((512, 4), (1024, 4), (2048, 4), (2048, 8)):
        t = graph_time(torch, lambda i: probe.read(views[i % nwin], blocks, unroll), 200, 5, reps=reps)
        best = t["median_ms"] if best is None else min(best, t["median_ms"])
    cache[key] = {"bytes": n, "us": round(best * 1e3, 2), "GBps": round(n / (best * 1e-3) / 1e9, 1)}
    return cache[key]


def bench_copy_probe(torch, reps):
    """Plain device-to-device copy of 1 GiB (read + write): the counter calibration kernel."""
    n = 1 << 29
    a = torch.empty(n, dtype=torch.float16, device=DEV).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    ms = statistics.median(_eager_ms(torch, lambda i: b.copy_(a), 100) for _ in range(reps))
    moved = 2 * a.numel() * a.element_size()
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_per_call": moved, "ms_per_call": round(ms, 6), "GBps": round(moved / (ms * 1e-3) / 1e9, 1),
            "timing": "eager back-to-back calls (0.4 ms each: host dispatch is hidden)"}


TRAFFIC = {}


def _roofline_hbm(gbps, kernel, nbytes, key, means):
    mean = means.get(key)
    r = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": round(gbps / HBM_PEAK_GBPS, 4), "kernel": kernel, "algorithmic_bytes_per_launch": nbytes,
         "rocprof_kernel_mean_us": mean, "traffic": TRAFFIC.get(key)}
    if mean:
        r["achieved_by_rocprof_mean"] = round(nbytes / (mean * 1e-6) / 1e9, 1)
        r["frac_by_rocprof_mean"] = round(r["achieved_by_rocprof_mean"] / HBM_PEAK_GBPS, 4)
    return r


def _finish_timing(res, t):
    res["ms_per_call"] = round(t["median_ms"], 6)
    res["ms_per_call_min"] = round(t["min_ms"], 6)
    res["rep_ms_per_call"] = t["rep_ms"]
    res["calls_per_rep"] = t["calls_per_rep"]
    res["graph_matches_eager"] = t["graph_matches_eager"]


def bench_decode(torch, gqa, synth, name, G, n_calls, warmup, reps, flusher, means, key,
                 append=False, dtype=None, keep_sample=False, direct_timing=False):
    w = synth.WORKLOADS[name]
    B, H, d, N = w.B, w.H, w.d, w.N
    dt = dtype or w.dtype
    itemsize = 4 if dt == "f32" else 2
    kv_bytes = 2 * B * G * N * d * itemsize
    R = 1 if w.seqlens == "uniform" else max(1, min(256, math.ceil((1 << 30) / kv_bytes)))
    make = synth.decode_append_inputs if append else synth.decode_inputs
    reps_in = [make(B, H, G, d, N, dtype=dt, seed=w.seed + r, device=DEV,
                    seqlens=w.seqlens, nan_tail=w.nan_tail) for r in range(R)]
    out = torch.empty_like(reps_in[0]["q"])
    S = gqa.decode_num_splits(B, H, G, d, N)
    # zero-filled once; the library leaves its counter header zero after each call
    ws = torch.zeros(max(gqa.decode_workspace_bytes(B, H, G, d, N), 1), dtype=torch.uint8, device=DEV)
    scale = synth.scale_for(d)

    def call(i):
        x = reps_in[i % R]
        if append:      # the same row is written again on every call: idempotent
            gqa.decode_append(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                              x["seqlens"], scale=scale, out=out, workspace=ws)
        else:
            gqa.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale, out=out,
                       workspace=ws)

    if n_calls is None:
        n_calls = calls_for(_eager_ms(torch, call, 20))
    t = graph_time(torch, call, n_calls, warmup, reps=reps, out=out)
    graph_ms = t["median_ms"]
    direct = None
    if not append:
        runs = flusher.probe.decode_call_loop(gqa, reps_in, out, ws, B, H, G, d, N, scale, n_calls,
                                              warmup=max(warmup, 1), reps=reps, lead=flusher.buf)
        direct = statistics.median(runs)
        if direct_timing:
            # the K steps timed as K direct calls queued behind the lead read
            t = dict(t, median_ms=direct, min_ms=min(runs), rep_ms=[round(x, 6) for x in runs])
    cold = flusher.latency_us(call, 0)
    total_pos = int(torch.clamp(reps_in[0]["seqlens"].long(), 0, N).sum().item())
    for r in reps_in[1:]:
        assert int(torch.clamp(r["seqlens"].long(), 0, N).sum().item()) == total_pos
    nbytes = decode_bytes(B, H, G, d, total_pos, itemsize)
    if append:          # the new rows: read from k_new/v_new and written into the caches
        nbytes += 2 * 2 * B * G * d * itemsize
    ms = t["median_ms"]
    gbps = round(nbytes / (ms * 1e-3) / 1e9, 1)
    res = {"B": B, "H": H, "G": G, "d": d, "N": N, "dtype": dt, "splits": S, "replicas": R,
           "replica_bytes": R * kv_bytes}
    _finish_timing(res, t)
    res.update({
        "bytes_per_call": nbytes, "split_partial_bytes": split_partial_bytes(B, H, d, S),
        "GBps": gbps, "GBps_at_min": round(nbytes / (t["min_ms"] * 1e-3) / 1e9, 1),
        "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(B / (ms * 1e-3), 1),
        "TFLOPs": round(decode_flops(H, total_pos, d) / (ms * 1e-3) / 1e12, 2),
        "cold_latency_us": cold,
        "direct_call_loop_ms_per_call": None if direct is None else round(direct, 6),
        "graph_replay_ms_per_call": round(graph_ms, 6),
        "roofline": _roofline_hbm(gbps, "decode_mfma_kernel" if dt != "f32" else "rows_valu_kernel",
                                  nbytes, key, means),
    })
    sample = None
    if keep_sample:
        # the GPU result of replica 0 and the inputs it came from, for the oracle
        call(0)
        torch.cuda.synchronize()
        sample = {"kind": "decode", "x": reps_in[0], "out": out.clone(), "scale": scale, "name": key}
        reps_in = [reps_in[0]]
    del reps_in
    torch.cuda.empty_cache()
    return res, sample


def bench_prefill(torch, gqa, synth, n_calls, warmup, reps, flusher, means, key, dtype=None,
                  keep_sample=False):
    w = synth.WORKLOADS["causal_prefill_bf16"]
    dt = dtype or w.dtype
    x = synth.prefill_inputs(w.B, w.N, w.H, w.G, w.d, dtype=dt, seed=w.seed, device=DEV, std=w.std)
    out = torch.empty_like(x["q"])
    scale = synth.scale_for(w.d)

    def call(i):
        gqa.prefill_causal(x["q"], x["k"], x["v"], scale=scale, out=out)

    if n_calls is None:
        n_calls = calls_for(_eager_ms(torch, call, 10))
    t = graph_time(torch, call, n_calls, warmup, reps=reps, out=out)
    cold = flusher.latency_us(call, 0)
    fl = prefill_flops(w.B, w.N, w.H, w.d)
    tf = round(fl / (t["median_ms"] * 1e-3) / 1e12, 1)
    res = {"B": w.B, "T": w.N, "H": w.H, "G": w.G, "d": w.d, "dtype": dt}
    _finish_timing(res, t)
    mean = means.get(key)
    res.update({
        "flops_per_call": fl, "TFLOPs": tf, "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
        "TFLOPs_at_min": round(fl / (t["min_ms"] * 1e-3) / 1e12, 1),
        "tokens_per_s": round(w.B * w.N / (t["median_ms"] * 1e-3), 1), "cold_latency_us": cold,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / BF16_PEAK_TFLOPS, 4), "kernel": "prefill_mfma_kernel",
                     "algorithmic_flops_per_launch": fl, "rocprof_kernel_mean_us": mean,
                     "traffic": TRAFFIC.get(key)},
    })
    if mean:
        res["roofline"]["achieved_by_rocprof_mean"] = round(fl / (mean * 1e-6) / 1e12, 1)
        res["roofline"]["frac_by_rocprof_mean"] = round(fl / (mean * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)
    sample = None
    if keep_sample:
        call(0)
        torch.cuda.synchronize()
        sample = {"kind": "prefill", "x": x, "out": out.clone(), "scale": scale, "name": key}
    else:
        del x
    del out
    torch.cuda.empty_cache()
    return res, sample


def bench_prefill_chunk(torch, gqa, synth, warmup, reps, means, key, ctx=2048, T=2048):
    """A T-token prompt chunk after ctx cached tokens (Llama-7B-sized layer, bf16)."""
    B, H, G, d = 2, 32, 8, 128
    n_max = ctx + T
    x = synth.decode_inputs(B, H, G, d, n_max, dtype="bf16", seed=21, device=DEV)
    q = synth.prefill_inputs(B, T, H, G, d, dtype="bf16", seed=22, device=DEV)["q"]
    cl = torch.full((B,), ctx, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    scale = synth.scale_for(d)

    def call(i):
        gqa.prefill_chunk(q, x["k_cache"], x["v_cache"], cl, scale=scale, out=out)

    t = graph_time(torch, call, calls_for(_eager_ms(torch, call, 10)), warmup, reps=reps, out=out)
    attended = B * H * (T * ctx + T * (T + 1) // 2)      # (row, key) pairs
    fl = 4 * d * attended
    tf = round(fl / (t["median_ms"] * 1e-3) / 1e12, 1)
    res = {"B": B, "T": T, "ctx": ctx, "H": H, "G": G, "d": d, "dtype": "bf16"}
    _finish_timing(res, t)
    res.update({"flops_per_call": fl, "TFLOPs": tf, "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tf / BF16_PEAK_TFLOPS, 4), "kernel": "prefill_mfma_kernel",
                             "rocprof_kernel_mean_us": means.get(key), "traffic": TRAFFIC.get(key)}})
    del x, q, out
    torch.cuda.empty_cache()
    return res


def bench_gqkva_decode(torch, gqa, synth, warmup, reps, means, key, g_q=4, g_kv=8):
    """GQKVA decode on the Llama-7B-sized cache: g_q query groups x g_kv K/V groups."""
    B, d, N = 16, 128, 1024
    kv_bytes = 2 * B * g_kv * N * d * 2
    R = max(1, min(256, math.ceil((1 << 30) / kv_bytes)))
    reps_in = [synth.decode_inputs(B, g_q, g_kv, d, N, dtype="bf16", seed=30 + r, device=DEV)
               for r in range(R)]
    out = torch.empty((B, g_q * g_kv, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(max(gqa.load_library().gqkva_decode_workspace_bytes(B, g_q, g_kv, d, N, 0), 1),
                     dtype=torch.uint8, device=DEV)
    scale = synth.scale_for(d)

    def call(i):
        x = reps_in[i % R]
        gqa.gqkva_decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale, out=out,
                         workspace=ws)

    t = graph_time(torch, call, calls_for(_eager_ms(torch, call, 20)), warmup, reps=reps, out=out)
    nbytes = 2 * B * g_kv * N * d * 2 + B * g_q * d * 2 + B * g_q * g_kv * d * 2 + 4 * B
    gbps = round(nbytes / (t["median_ms"] * 1e-3) / 1e9, 1)
    res = {"B": B, "g_q": g_q, "g_kv": g_kv, "d": d, "N": N, "dtype": "bf16", "replicas": R}
    _finish_timing(res, t)
    res.update({"bytes_per_call": nbytes, "GBps": gbps, "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                "roofline": _roofline_hbm(gbps, "decode_mfma_kernel", nbytes, key, means)})
    del reps_in
    torch.cuda.empty_cache()
    return res


def bench_meanpool(torch, gqa, synth, warmup, reps, means, key, keep_sample=False):
    w = synth.WORKLOADS["t5xxl_meanpool_bf16"]
    per_head = 1
    for s in w.per_head_shape:
        per_head *= s
    in_bytes = w.H * per_head * 2
    R = max(1, min(256, math.ceil((1 << 30) / in_bytes)))
    reps_in = [synth.meanpool_inputs(w.H, w.per_head_shape, dtype=w.dtype, seed=r, device=DEV)["w"]
               for r in range(R)]
    out = torch.empty((w.G,) + tuple(w.per_head_shape), dtype=reps_in[0].dtype, device=DEV)

    def call(i):
        gqa.meanpool_heads(reps_in[i % R], w.G, out=out)

    t = graph_time(torch, call, calls_for(_eager_ms(torch, call, 20)), warmup, reps=reps, out=out)
    nbytes = (w.H + w.G) * per_head * 2
    gbps = round(nbytes / (t["median_ms"] * 1e-3) / 1e9, 1)
    res = {"H": w.H, "G": w.G, "per_head_shape": list(w.per_head_shape), "replicas": R}
    _finish_timing(res, t)
    res.update({"bytes_per_call": nbytes, "GBps": gbps, "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                "roofline": _roofline_hbm(gbps, "meanpool_vec8_kernel", nbytes, key, means)})
    sample = None
    if keep_sample:
        call(0)
        torch.cuda.synchronize()
        sample = {"kind": "meanpool", "w": reps_in[0], "G": w.G, "out": out.clone(), "name": key}
    del reps_in
    torch.cuda.empty_cache()
    return res, sample


def bench_meanpool_batch(torch, gqa, synth, count, warmup, reps, means, key):
    """kv_meanpool_heads_batch over `count` T5-XXL projections per call (count
    = 2: one layer's K and V; 16: eight layers'), timed per call; the rate
    and roofline count every projection's bytes."""
    w = synth.WORKLOADS["t5xxl_meanpool_bf16"]
    per_head = 1
    for s in w.per_head_shape:
        per_head *= s
    in_bytes = w.H * per_head * 2
    R = max(1, min(256, math.ceil((1 << 30) / (count * in_bytes))))
    reps_in = [[synth.meanpool_inputs(w.H, w.per_head_shape, dtype=w.dtype, seed=1000 * r + j, device=DEV)["w"]
                for j in range(count)] for r in range(R)]
    outs = [torch.empty((w.G,) + tuple(w.per_head_shape), dtype=reps_in[0][0].dtype, device=DEV)
            for _ in range(count)]

    def call(i):
        gqa.meanpool_heads_batch(reps_in[i % R], w.G, outs=outs)

    t = graph_time(torch, call, calls_for(_eager_ms(torch, call, 20)), warmup, reps=reps, out=outs[-1])
    nbytes = count * (w.H + w.G) * per_head * 2
    gbps = round(nbytes / (t["median_ms"] * 1e-3) / 1e9, 1)
    res = {"H": w.H, "G": w.G, "per_head_shape": list(w.per_head_shape), "projections_per_call": count,
           "replicas": R}
    _finish_timing(res, t)
    res.update({"us_per_projection": round(t["median_ms"] * 1e3 / count, 3), "bytes_per_call": nbytes,
                "GBps": gbps, "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                "roofline": _roofline_hbm(gbps, "meanpool_vec8_kernel", nbytes, key, means)})
    del reps_in
    torch.cuda.empty_cache()
    return res


class _Progress(dict):
    """The secondary results; each workload's time goes to stderr as it finishes (a progress line)."""

    def __setitem__(self, key, value):
        super().__setitem__(key, value)
        if isinstance(value, dict):
            t = value.get("ms_per_call")
            msg = f"{t * 1e3:.2f} us per call" if t is not None else "done"
            print(f"[bench] {key}: {msg}", file=sys.stderr, flush=True)


def g_sweep_fit(points):
    """Least-squares line time = fixed + bytes / bandwidth over the G sweep."""
    xs = [p["bytes_per_call"] for p in points]
    ys = [p["ms_per_call"] * 1e-3 for p in points]
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    slope = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx
    icpt = my - slope * mx
    return {"fixed_us": round(icpt * 1e6, 2), "marginal_GBps": round(1 / slope / 1e9, 1),
            "points": {f"G{p['G']}": {"MB": round(p["bytes_per_call"] / 1e6, 2),
                                      "us": round(p["ms_per_call"] * 1e3, 2)} for p in points}}


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host cores, and the GPU's errors
# ---------------------------------------------------------------------------

def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            i = info[0]
            return {"vendor": i.get("internal_api"), "version": i.get("version"),
                    "threads": int(i.get("num_threads", 1))}
    except Exception:   # pragma: no cover
        pass
    return {"vendor": "unknown", "version": None, "threads": os.cpu_count() or 1}


def _err_stats(got, ref, dtype_name):
    """Max and mean absolute error against the float64 oracle; for 16-bit
    outputs also the largest error in units of the output format's ulp at the
    oracle value, over outputs with |oracle| >= 1/4 (where a rounding of the
    output, up to half an ulp, is the size of the absolute tolerance; near
    zero an ulp count says nothing), and the fraction of all outputs equal to
    the oracle rounded to nearest even."""
    import numpy as np
    import torch
    g = got.detach().to("cpu", torch.float32).numpy().astype(np.float64)
    e = np.abs(g - ref)
    st = {"max_abs": float(e.max(initial=0.0)), "mean_abs": float(e.mean()) if e.size else 0.0}
    if dtype_name in ("bf16", "f16"):
        tdt, frac_bits = (torch.bfloat16, 7) if dtype_name == "bf16" else (torch.float16, 10)
        big = np.abs(ref) >= 0.25
        ulp = np.exp2(np.floor(np.log2(np.abs(ref[big]))) - frac_bits)
        want = torch.from_numpy(ref.astype(np.float32)).to(tdt).view(torch.int16).numpy()
        have = got.detach().cpu().view(torch.int16).numpy()
        st["max_err_ulps_at_oracle_abs_ge_0.25"] = float((e[big] / ulp).max(initial=0.0))
        st["frac_equal_rne_oracle"] = float((want == have).mean()) if e.size else 1.0
    return {k: (round(v, 8) if isinstance(v, float) else v) for k, v in st.items()}


def cpu_baseline(torch, samples, budget_s):
    """Time the oracle on each workload's sample (bounded), compare the GPU output."""
    import numpy as np
    import oracle
    blas = _blas_info()
    to64 = lambda t: t.detach().to("cpu", torch.float32).numpy().astype(np.float64)   # noqa: E731
    per = {}
    head = None
    for s in samples:
        name = s["name"]
        t0 = time.perf_counter()
        if s["kind"] == "decode":
            x = s["x"]
            B, H, d = x["q"].shape
            G, n_max = x["k_cache"].shape[1], x["k_cache"].shape[2]
            sl = x["seqlens"].cpu().numpy()
            itemsize = x["q"].element_size()
            if name == HEADLINE_KEY:
                # the headline: whole calls, repeated for about budget_s
                q, k, v = to64(x["q"]), to64(x["k_cache"]), to64(x["v_cache"])
                t0 = time.perf_counter()
                calls = 0
                while True:
                    ref = oracle.decode_ref(q, k, v, sl, s["scale"])
                    calls += 1
                    if time.perf_counter() - t0 >= budget_s:
                        break
                dt = time.perf_counter() - t0
                nb = decode_bytes(B, H, G, d, int(np.clip(sl, 0, n_max).sum()), itemsize) * calls
                head = {"value": round(nb / dt / 1e9, 4), "unit": "GB/s", "calls": calls, "seconds": dt}
                rows = list(range(B))
                got = s["out"]
            else:
                # at most 4 sequences, only their attended rows copied to the host
                rows = list(range(B)) if B * G * n_max * d <= (1 << 26) else list(range(min(B, 4)))
                refs, pos = [], 0
                t0 = time.perf_counter()
                for b in rows:
                    n = int(min(max(int(sl[b]), 0), n_max))
                    kk = to64(x["k_cache"][b:b + 1, :, :max(n, 1)])
                    vv = to64(x["v_cache"][b:b + 1, :, :max(n, 1)])
                    refs.append(oracle.decode_ref(to64(x["q"][b:b + 1]), kk, vv, [sl[b]], s["scale"])[0])
                    pos += n
                dt = time.perf_counter() - t0
                ref = np.stack(refs)
                got = s["out"][rows]
                nb = decode_bytes(len(rows), H, G, d, pos, itemsize)
            per[name] = {"seconds": round(dt, 3), "GBps": round(nb / dt / 1e9, 4),
                         "sample": f"{len(rows)} of {B} sequences",
                         "gpu_vs_oracle": _err_stats(got, ref, "bf16" if itemsize == 2 and
                                                     x["q"].dtype == torch.bfloat16 else
                                                     ("f16" if itemsize == 2 else "f32"))}
        elif s["kind"] == "prefill":
            x = s["x"]
            B, T, H, d = x["q"].shape
            G = x["k"].shape[2]
            # one sequence, every 4th row (the keys of all T positions are still read)
            rows = np.arange(0, T, 4)
            t0 = time.perf_counter()
            ref = oracle.prefill_causal_ref(to64(x["q"][:1]), to64(x["k"][:1]), to64(x["v"][:1]),
                                            s["scale"], rows=rows)
            dt = time.perf_counter() - t0
            fl = 4 * d * H * int((rows + 1).sum())      # algorithmic flops of those rows
            per[name] = {"seconds": round(dt, 3), "GFLOPs": round(fl / dt / 1e9, 3),
                         "sample": f"sequence 0, {len(rows)} of {T} rows (every 4th), all {H} heads; "
                                   "the oracle scores every key of a row and masks (2x the causal flops)",
                         "gpu_vs_oracle": _err_stats(s["out"][:1, torch.as_tensor(rows, device=s["out"].device)],
                                                     ref[:, rows], "bf16")}
        elif s["kind"] == "meanpool":
            w = s["w"]
            t0 = time.perf_counter()
            ref = oracle.meanpool_ref(to64(w), s["G"])
            dt = time.perf_counter() - t0
            nb = (w.shape[0] + s["G"]) * w[0].numel() * w.element_size()
            per[name] = {"seconds": round(dt, 3), "GBps": round(nb / dt / 1e9, 4), "sample": "whole call",
                         "gpu_vs_oracle": _err_stats(s["out"], ref, "bf16")}
    if head is None:
        return None
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": head["value"], "unit": "GB/s", "cores": blas["threads"], "kind": "oracle",
            "sample": f"{head['calls']} whole calls of the headline decode step ({HEADLINE_KEY}), "
                      f"bf16 values upcast to float64 arithmetic, {head['seconds']:.1f} s",
            "host_cores_available": cores, "blas": blas, "per_workload": per}


HEADLINE_KEY = "llama7b_decode_G8"


# ---------------------------------------------------------------------------
# --timeline: per-workgroup phases of the matrix-core decode (libgqa_timeline.so)
# ---------------------------------------------------------------------------

TIMELINE_WORKLOADS = [("llama7b_decode_bf16", 8), ("llama7b_decode_bf16", 1), ("llama7b_decode_bf16", 4),
                      ("llama7b_decode_bf16", 32), ("t5xxl_cross_decode_bf16", 8)]
TICK_US = 0.01          # the device clock read by the timeline build runs at 100 MHz


def _by_xcd(t, rows, col):
    """Median of phase ``col`` over the workgroups of each XCD (slot 7 of the timeline)."""
    import numpy as np
    out = {}
    for x in range(8):
        vals = np.concatenate([r[t[c][t[c][:, 0] != 0][:, 7] == x, col] for c, r in enumerate(rows)])
        vals = vals[~np.isnan(vals)]
        if vals.size:
            out[str(x)] = round(float(np.median(vals)), 2)
    return out


def timeline(torch, synth, n_calls=40):
    """Phase timestamps of every workgroup over n_calls graph-replayed decode calls.

    Per workgroup: 0 start, 1 length known, 2 first tile done, 3 tile loop done,
    4 partial (or output) stored and acknowledged, 5 arrival counted, 6 end;
    times are taken relative to the earliest start of the same call."""
    import numpy as np
    import grouped_query_decode_amd as gqa
    path = os.path.join(os.path.dirname(gqa.library_path()), "libgqa_timeline.so")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gqa_decode_split.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, sz, vp]
    lib.gqa_decode_split.restype = i32
    lib.gqa_timeline_set_buffer.argtypes = [vp]
    lib.gqa_decode_num_splits.argtypes = [i32] * 5
    lib.gqa_decode_workspace_bytes.argtypes = [i32] * 6
    lib.gqa_decode_workspace_bytes.restype = sz
    result = {}
    for name, G in TIMELINE_WORKLOADS:
        w = synth.WORKLOADS[name]
        B, H, d, N = w.B, w.H, w.d, w.N
        kv_bytes = 2 * B * G * N * d * 2
        R = max(1, min(256, math.ceil((1 << 30) / kv_bytes)))
        reps_in = [synth.decode_inputs(B, H, G, d, N, dtype="bf16", seed=w.seed + r, device=DEV) for r in range(R)]
        out = torch.empty_like(reps_in[0]["q"])
        ws = torch.zeros(max(int(lib.gqa_decode_workspace_bytes(B, H, G, d, N, 0)), 1), dtype=torch.uint8,
                         device=DEV)
        S = int(lib.gqa_decode_num_splits(B, H, G, d, N))
        grid_max = B * G * S * 2
        tl = torch.zeros((n_calls, grid_max, 8), dtype=torch.int64, device=DEV)
        stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)   # noqa: E731

        def call(i, buf):
            x = reps_in[i % R]
            lib.gqa_timeline_set_buffer(ctypes.c_void_p(buf))
            st = lib.gqa_decode_split(ctypes.c_void_p(x["q"].data_ptr()), ctypes.c_void_p(x["k_cache"].data_ptr()),
                                      ctypes.c_void_p(x["v_cache"].data_ptr()),
                                      ctypes.c_void_p(x["seqlens"].data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                      B, H, G, d, N, synth.scale_for(d), 1, 0, ctypes.c_void_p(ws.data_ptr()),
                                      ws.numel(), stream())
            assert st == 0, st

        for i in range(20):
            call(i, None)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_calls):
                call(i, tl[i].data_ptr())
        lib.gqa_timeline_set_buffer(None)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tl.zero_()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ev_us = a.elapsed_time(b) * 1e3 / n_calls
        t = tl.cpu().numpy()
        rows = []
        for c in range(n_calls):
            used = t[c][t[c][:, 0] != 0]
            t0 = used[:, 0].min()
            rel = (used[:, :7] - t0).astype(np.float64) * TICK_US
            rel[used[:, :7] == 0] = np.nan
            rows.append(rel)
        def phase(col):
            """Median over calls of the median and of the latest workgroup of phase col."""
            meds, maxs = [], []
            for r in rows:
                v = r[:, col]
                v = v[~np.isnan(v)]
                if v.size:
                    meds.append(float(np.median(v)))
                    maxs.append(float(v.max()))
            if not meds:
                return None
            return {"median": round(float(np.median(meds)), 2), "latest": round(float(np.median(maxs)), 2)}

        # the merging workgroup of a (b, g) is the one whose end comes long
        # after its count (the others end right after counting in): per call,
        # the longest count-to-end span is the slowest merge
        merges = []
        for r in rows:
            both = r[~np.isnan(r[:, 5]) & ~np.isnan(r[:, 6])]
            if len(both):
                merges.append(float(np.max(both[:, 6] - both[:, 5])))
        result[f"{name}:G{G}"] = {
            "workgroups": int(np.sum(t[0][:, 0] != 0)), "splits": S, "event_us_per_call": round(ev_us, 2),
            "started": phase(0), "length_known": phase(1), "first_tile_done": phase(2),
            "loop_done": phase(3), "stored": phase(4), "counted": phase(5), "end": phase(6),
            "slowest_merge_us": round(float(np.median(merges)), 2) if merges else None,
            "loop_done_median_by_xcd": _by_xcd(t, rows, 3),
        }
        del reps_in, tl, g
        torch.cuda.empty_cache()
    return result


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4000, help="calls per timed replay of the headline")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--reps", type=int, default=REPS)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--only", default="", help="comma-separated secondary workload keys")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--probe-rates", action="store_true",
                    help="print the vector-unit issue rates (fma, exp) and LDS read rates, and exit")
    ap.add_argument("--timeline", action="store_true",
                    help="print per-workgroup decode phase timings (libgqa_timeline.so) instead of the bench line")
    ap.add_argument("--min-rep-ms", type=float, default=50.0,
                    help="minimum length of a timed replay of a secondary workload (profiling runs lower it)")
    args = ap.parse_args()
    global MIN_REP_MS
    MIN_REP_MS = args.min_rep_ms

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the decode, prefill and "
                                   "mean-pool kernels are single-GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import grouped_query_decode_amd as gqa
    import synth

    gqa.load_library()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    if args.timeline:
        print(json.dumps({"decode_timeline": timeline(torch, synth)}), flush=True)
        return
    probe = ReadProbe(torch)
    if args.probe_rates:
        print(json.dumps({"valu_issue_rates": probe.valu_rates(), "lds_read_rates": probe.lds_rates()}),
              flush=True)
        return
    flusher = ColdFlusher(torch, probe)
    global LEAD
    LEAD = flusher.lead
    means = stored_kernel_means()
    TRAFFIC.update(stored_traffic())
    want_cpu = not args.no_cpu_baseline
    only = set(filter(None, args.only.split(",")))
    run = (lambda k: (not args.quick) and (not only or k in only))   # noqa: E731
    samples = []
    reps = args.reps

    name, G = HEADLINE
    # K steps are timed as a graph replay when K >= MIN_CALLS (the replay's fixed
    # ~10 us of device-side cost is then amortised), else as K direct calls from
    # C queued behind the lead read (no per-replay cost, ~0.1 us more per call)
    direct_headline = args.steps < MIN_CALLS
    head, s = bench_decode(torch, gqa, synth, name, G, args.steps, args.warmup, reps, flusher, means,
                           HEADLINE_KEY, keep_sample=want_cpu, direct_timing=direct_headline)
    if s:
        samples.append(s)
    print(f"[bench] {HEADLINE_KEY}: {head['ms_per_call'] * 1e3:.2f} us per call", file=sys.stderr, flush=True)
    secondary = _Progress()
    sweep = [head]
    for g in (32, 4, 1):
        k = f"llama7b_decode_G{g}"
        if run(k) or run("g_sweep"):
            secondary[k], _ = bench_decode(torch, gqa, synth, name, g, None, args.warmup, reps, flusher,
                                           means, k)
            sweep.append(secondary[k])
    if len(sweep) == 4:
        secondary["g_sweep_fit"] = g_sweep_fit(sorted(sweep, key=lambda p: p["G"]))
    if run("tiny_decode_f32"):
        w = synth.WORKLOADS["tiny_decode_f32"]
        for g in w.G_sweep:
            k = f"tiny_decode_f32_G{g}"
            secondary[k], s = bench_decode(torch, gqa, synth, "tiny_decode_f32", g, None, args.warmup, reps,
                                           flusher, means, k, keep_sample=want_cpu and g == w.G)
            if s:
                samples.append(s)
    if run("llama7b_decode_append_G8"):
        secondary["llama7b_decode_append_G8"], _ = bench_decode(
            torch, gqa, synth, name, 8, None, args.warmup, reps, flusher, means, "llama7b_decode_append_G8",
            append=True)
    if run("t5xxl_cross_decode"):
        secondary["t5xxl_cross_decode"], s = bench_decode(
            torch, gqa, synth, "t5xxl_cross_decode_bf16", 8, None, args.warmup, reps, flusher, means,
            "t5xxl_cross_decode", keep_sample=want_cpu)
        if s:
            samples.append(s)
    if run("ragged_longctx_decode"):
        secondary["ragged_longctx_decode"], s = bench_decode(
            torch, gqa, synth, "ragged_longctx_decode_bf16", 8, None, 3, reps, flusher, means,
            "ragged_longctx_decode", keep_sample=want_cpu)
        if s:
            samples.append(s)
    if run("llama7b_decode_G8_f16"):
        secondary["llama7b_decode_G8_f16"], _ = bench_decode(
            torch, gqa, synth, name, 8, None, args.warmup, reps, flusher, means, "llama7b_decode_G8_f16",
            dtype="f16")
    if run("gqkva_decode_q4_kv8"):
        secondary["gqkva_decode_q4_kv8"] = bench_gqkva_decode(torch, gqa, synth, args.warmup, reps, means,
                                                              "gqkva_decode_q4_kv8")
    if run("t5xxl_meanpool"):
        secondary["t5xxl_meanpool"], s = bench_meanpool(torch, gqa, synth, args.warmup, reps, means,
                                                        "t5xxl_meanpool", keep_sample=want_cpu)
        if s:
            samples.append(s)
    for count, k in ((2, "t5xxl_meanpool_kv_layer"), (16, "t5xxl_meanpool_8_layers_kv")):
        if run(k):
            secondary[k] = bench_meanpool_batch(torch, gqa, synth, count, args.warmup, reps, means, k)
    # prefill runs the matrix cores flat out: its first ~20 calls after the
    # memory-bound work run ~20% slower while the clock ramps up, so it gets
    # PREFILL_WARMUP untimed calls (about 35 ms) first
    if run("causal_prefill"):
        secondary["causal_prefill"], s = bench_prefill(torch, gqa, synth, None, PREFILL_WARMUP, reps, flusher,
                                                       means, "causal_prefill", keep_sample=want_cpu)
        if s:
            samples.append(s)
    if run("causal_prefill_f16"):
        secondary["causal_prefill_f16"], _ = bench_prefill(torch, gqa, synth, None, PREFILL_WARMUP, reps,
                                                           flusher, means, "causal_prefill_f16", dtype="f16")
    if run("prefill_chunk_2048_after_2048"):
        secondary["prefill_chunk_2048_after_2048"] = bench_prefill_chunk(
            torch, gqa, synth, PREFILL_WARMUP, reps, means, "prefill_chunk_2048_after_2048")
    if run("hbm_copy_probe"):
        secondary["hbm_copy_probe"] = bench_copy_probe(torch, reps)
    ceiling = None
    if run("hbm_read_probe"):
        secondary["hbm_read_probe"] = bench_read_probe(torch, probe, reps)
        ceiling = secondary["hbm_read_probe"]["GBps"]
    if ceiling:
        sized = {}
        for v in [head] + list(secondary.values()):
            if isinstance(v, dict) and "roofline" in v and v["roofline"]["bound"] == "hbm":
                r = v["roofline"]
                r["frac_of_measured_read_ceiling"] = round(v["GBps"] / ceiling, 4)
                at = probe_at_size(torch, probe, v["bytes_per_call"], reps, sized)
                # beyond the probe's 2 GiB buffer the rate no longer depends on size: the
                # workload's bytes at that rate
                r["read_probe_at_same_bytes"] = {
                    "us": round(v["bytes_per_call"] / (at["GBps"] * 1e3), 2), "GBps": at["GBps"],
                    "bytes_probed": at["bytes"]}
                r["frac_of_read_probe_at_same_bytes"] = round(v["GBps"] / at["GBps"], 4)
        sized.pop("buf", None)
        torch.cuda.empty_cache()

    if not args.quick and not only:
        secondary["valu_issue_rates"] = probe.valu_rates()
    roofline = dict(head["roofline"])
    roofline["kernel"] = ("decode_mfma_kernel<128,1>" +
                          (" (split merge fused)" if head["splits"] > 1 else " (one split per (b, g))"))
    line = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": head["calls_per_rep"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": head["B"], "H": head["H"], "G": G, "d": head["d"],
                   "N": head["N"], "splits": head["splits"], "replicas": head["replicas"]},
        "timing": {"method": ("`steps` back-to-back calls of the C entry point made directly from C, "
                              "queued behind a 1 GiB device read (so the events bracket exactly the calls), "
                              "`reps` runs; median per call") if direct_headline else
                             ("HIP graph of `steps` calls, replayed `reps` times behind a 1 GiB device read; "
                              "median per call"),
                   "reps": reps, "ms_per_step_min": head["ms_per_call_min"],
                   "rep_ms_per_step": head["rep_ms_per_call"],
                   "graph_replay_ms_per_step": head["graph_replay_ms_per_call"],
                   "direct_call_loop_ms_per_step": head["direct_call_loop_ms_per_call"],
                   "graph_matches_eager": head["graph_matches_eager"],
                   "cold_latency_us": head["cold_latency_us"]},
        "tokens_per_s": head["tokens_per_s"],
        "roofline": roofline,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "gcn_arch": getattr(props, "gcnArchName", "")},
        "secondary": secondary,
    }
    if want_cpu:
        line["cpu_baseline"] = cpu_baseline(torch, samples, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
