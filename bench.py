"""Benchmark of the GQA hot path on one MI355X; prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu-baseline]

Headline (``value``): KV-read GB/s of one GQA decode step on the Llama-7B-sized
layer (B=16, H=32 query heads, G=8 K/V heads, d=128, cache length 1024, bf16),
i.e. algorithmic bytes (K and V actually attended, plus q and out) divided by
the measured time per call.  Inputs are resident in HBM; every call reads a
different replica of the cache, rotating over >= 1 GiB of replicas, so the
256 MB last-level cache cannot serve a call from the previous one.

Also reported (``secondary``): the G sweep {32, 8, 4, 1} on the same queries,
the T5-XXL-sized cross-attention step, the ragged 32k-context step, the causal
prefill (TFLOP/s against the bf16 matrix peak) and the K/V mean-pool.  The
float64 oracle is timed on the host cores on a bounded sample of the headline
workload (``cpu_baseline``).  A step is one call of the library entry point.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published
PREFILL_WARMUP = 120              # untimed prefill calls before timing (clock ramp-up)
BF16_PEAK_TFLOPS = 2500.0         # MI355X dense bf16 matrix, published
HEADLINE = ("llama7b_decode_bf16", 8)
METRIC = "decode KV-read GB/s (% of HBM peak) + tokens/s; prefill TFLOP/s (% MFMA)"
DECODE_KERNEL_SOURCES = ["grouped_query_decode_amd/csrc/decode_mfma.hip",
                         "grouped_query_decode_amd/csrc/device_common.h",
                         "grouped_query_decode_amd/csrc/internal.h",
                         "grouped_query_decode_amd/csrc/api.cpp"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_llama7b_G8_hbm_counters.md")


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


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in DECODE_KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch from the committed counter summary, if still current."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_val or m_sha.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def _time_calls(torch, fn, n_calls, warmup):
    """Average milliseconds per call over n_calls back-to-back calls (events on the launch stream)."""
    for i in range(warmup):
        fn(i)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(n_calls):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n_calls


def bench_decode(torch, gqa, synth, name, G, steps, warmup, replicas_bytes=1 << 30, append=False,
                 dtype=None):
    w = synth.WORKLOADS[name]
    B, H, d, N = w.B, w.H, w.d, w.N
    dt = dtype or w.dtype
    dev = "cuda:0"
    itemsize = 4 if dt == "f32" else 2
    kv_bytes = 2 * B * G * N * d * itemsize
    R = 1 if w.seqlens == "uniform" else max(1, min(64, math.ceil(replicas_bytes / kv_bytes)))
    make = synth.decode_append_inputs if append else synth.decode_inputs
    reps = [make(B, H, G, d, N, dtype=dt, seed=w.seed + r, device=dev,
                 seqlens=w.seqlens, nan_tail=w.nan_tail) for r in range(R)]
    q = reps[0]["q"]
    out = torch.empty_like(q)
    # zero-filled once; the library leaves its counter header zero after each call
    ws = torch.zeros(max(gqa.decode_workspace_bytes(B, H, G, d, N), 1), dtype=torch.uint8, device=dev)
    scale = synth.scale_for(d)

    def call(i):
        x = reps[i % R]
        if append:      # the same row is written again on every call: idempotent
            gqa.decode_append(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                              x["seqlens"], scale=scale, out=out, workspace=ws)
        else:
            gqa.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale, out=out,
                       workspace=ws)

    ms = _time_calls(torch, call, steps, warmup)
    total_pos = int(torch.clamp(reps[0]["seqlens"].long(), 0, N).sum().item())
    for r in reps[1:]:
        assert int(torch.clamp(r["seqlens"].long(), 0, N).sum().item()) == total_pos
    nbytes = decode_bytes(B, H, G, d, total_pos, itemsize)
    if append:          # the new rows: read from k_new/v_new and written into the caches
        nbytes += 2 * 2 * B * G * d * itemsize
    gbps = nbytes / (ms * 1e-3) / 1e9
    res = {
        "B": B, "H": H, "G": G, "d": d, "N": N, "dtype": dt,
        "splits": gqa.decode_num_splits(B, H, G, d, N), "replicas": R,
        "ms_per_call": round(ms, 6), "bytes_per_call": nbytes,
        "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(B / (ms * 1e-3), 1),
        "TFLOPs": round(decode_flops(H, total_pos, d) / (ms * 1e-3) / 1e12, 2),
    }
    del reps
    torch.cuda.empty_cache()
    return res


def bench_prefill(torch, gqa, synth, steps, warmup, dtype=None):
    w = synth.WORKLOADS["causal_prefill_bf16"]
    dt = dtype or w.dtype
    x = synth.prefill_inputs(w.B, w.N, w.H, w.G, w.d, dtype=dt, seed=w.seed,
                             device="cuda:0", std=w.std)
    out = torch.empty_like(x["q"])
    scale = synth.scale_for(w.d)
    ms = _time_calls(torch, lambda i: gqa.prefill_causal(x["q"], x["k"], x["v"], scale=scale, out=out),
                     steps, warmup)
    fl = prefill_flops(w.B, w.N, w.H, w.d)
    tf = fl / (ms * 1e-3) / 1e12
    del x, out
    torch.cuda.empty_cache()
    return {"B": w.B, "T": w.N, "H": w.H, "G": w.G, "d": w.d, "dtype": dt,
            "ms_per_call": round(ms, 6), "flops_per_call": fl, "TFLOPs": round(tf, 1),
            "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1)}


def bench_prefill_chunk(torch, gqa, synth, steps, warmup, ctx=2048, T=2048):
    """A T-token prompt chunk after ctx cached tokens (Llama-7B-sized layer, bf16)."""
    B, H, G, d = 2, 32, 8, 128
    n_max = ctx + T
    dev = "cuda:0"
    x = synth.decode_inputs(B, H, G, d, n_max, dtype="bf16", seed=21, device=dev)
    q = synth.prefill_inputs(B, T, H, G, d, dtype="bf16", seed=22, device=dev)["q"]
    cl = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    scale = synth.scale_for(d)
    ms = _time_calls(torch, lambda i: gqa.prefill_chunk(q, x["k_cache"], x["v_cache"], cl, scale=scale,
                                                        out=out), steps, warmup)
    attended = B * H * (T * ctx + T * (T + 1) // 2)      # (row, key) pairs
    fl = 4 * d * attended
    tf = fl / (ms * 1e-3) / 1e12
    del x, q, out
    torch.cuda.empty_cache()
    return {"B": B, "T": T, "ctx": ctx, "H": H, "G": G, "d": d, "dtype": "bf16",
            "ms_per_call": round(ms, 6), "flops_per_call": fl, "TFLOPs": round(tf, 1),
            "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}


def bench_gqkva_decode(torch, gqa, synth, steps, warmup, g_q=4, g_kv=8):
    """GQKVA decode on the Llama-7B-sized cache: g_q query groups x g_kv K/V groups."""
    B, d, N = 16, 128, 1024
    dev = "cuda:0"
    kv_bytes = 2 * B * g_kv * N * d * 2
    R = max(1, min(64, math.ceil((1 << 30) / kv_bytes)))
    reps = [synth.decode_inputs(B, g_q, g_kv, d, N, dtype="bf16", seed=30 + r, device=dev) for r in range(R)]
    out = torch.empty((B, g_q * g_kv, d), dtype=torch.bfloat16, device=dev)
    scale = synth.scale_for(d)
    ms = _time_calls(torch, lambda i: gqa.gqkva_decode(reps[i % R]["q"], reps[i % R]["k_cache"],
                                                       reps[i % R]["v_cache"], reps[i % R]["seqlens"],
                                                       scale=scale, out=out), steps, warmup)
    nbytes = 2 * B * g_kv * N * d * 2 + B * g_q * d * 2 + B * g_q * g_kv * d * 2 + 4 * B
    gbps = nbytes / (ms * 1e-3) / 1e9
    del reps
    torch.cuda.empty_cache()
    return {"B": B, "g_q": g_q, "g_kv": g_kv, "d": d, "N": N, "dtype": "bf16", "replicas": R,
            "ms_per_call": round(ms, 6), "bytes_per_call": nbytes, "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def bench_meanpool(torch, gqa, synth, steps, warmup):
    w = synth.WORKLOADS["t5xxl_meanpool_bf16"]
    per_head = 1
    for s in w.per_head_shape:
        per_head *= s
    in_bytes = w.H * per_head * 2
    R = max(1, min(64, math.ceil((1 << 30) / in_bytes)))
    reps = [synth.meanpool_inputs(w.H, w.per_head_shape, dtype=w.dtype, seed=r, device="cuda:0")["w"]
            for r in range(R)]
    out = torch.empty((w.G,) + tuple(w.per_head_shape), dtype=reps[0].dtype, device="cuda:0")
    ms = _time_calls(torch, lambda i: gqa.meanpool_heads(reps[i % R], w.G, out=out), steps, warmup)
    nbytes = (w.H + w.G) * per_head * 2
    gbps = nbytes / (ms * 1e-3) / 1e9
    del reps
    torch.cuda.empty_cache()
    return {"H": w.H, "G": w.G, "per_head_shape": list(w.per_head_shape), "replicas": R,
            "ms_per_call": round(ms, 6), "bytes_per_call": nbytes, "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def bench_read_probe(torch, steps):
    """Sum of a 2 GiB bf16 tensor (PyTorch's reduction): an achievable-read-bandwidth reference."""
    a = torch.ones(1 << 30, dtype=torch.bfloat16, device="cuda:0")
    ms = _time_calls(torch, lambda i: a.sum(dtype=torch.float32), max(5, steps // 10), 3)
    moved = a.numel() * a.element_size()
    del a
    torch.cuda.empty_cache()
    return {"bytes_per_call": moved, "ms_per_call": round(ms, 6),
            "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}


def bench_copy_probe(torch, steps):
    """Plain device-to-device copy of 1 GiB (read + write) as an achievable-bandwidth reference."""
    n = 1 << 29
    a = torch.empty(n, dtype=torch.float16, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    ms = _time_calls(torch, lambda i: b.copy_(a), max(5, steps // 10), 3)
    moved = 2 * a.numel() * a.element_size()
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_per_call": moved, "ms_per_call": round(ms, 6),
            "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host cores
# ---------------------------------------------------------------------------

def cpu_baseline(torch, synth, budget_s=12.0):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:   # pragma: no cover
        threads = os.cpu_count() or 1
    name, G = HEADLINE
    w = synth.WORKLOADS[name]
    x = synth.decode_inputs(w.B, w.H, G, w.d, w.N, dtype=w.dtype, seed=w.seed, device="cpu")
    q = x["q"].float().numpy()
    k = x["k_cache"].float().numpy()
    v = x["v_cache"].float().numpy()
    sl = x["seqlens"].numpy()
    scale = synth.scale_for(w.d)
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode_ref(q, k, v, sl, scale)
        calls += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    nbytes = decode_bytes(w.B, w.H, G, w.d, int(sl.sum()), 2)
    return {"value": round(nbytes * calls / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{calls} full calls of the headline decode step (B={w.B}, H={w.H}, G={G}, "
                      f"d={w.d}, N={w.N}; bf16 values as float32 arrays, float64 arithmetic), "
                      f"{dt:.1f} s",
            "s_per_call": round(dt / calls, 4)}


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    args = ap.parse_args()

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

    name, G = HEADLINE
    head = bench_decode(torch, gqa, synth, name, G, args.steps, args.warmup)
    secondary = {}
    if not args.quick:
        for g in (32, 4, 1):
            secondary[f"llama7b_decode_G{g}"] = bench_decode(torch, gqa, synth, name, g, args.steps, args.warmup)
        secondary["llama7b_decode_append_G8"] = bench_decode(torch, gqa, synth, name, 8, args.steps,
                                                              args.warmup, append=True)
        secondary["t5xxl_cross_decode"] = bench_decode(torch, gqa, synth, "t5xxl_cross_decode_bf16", 8,
                                                       args.steps, args.warmup)
        secondary["ragged_longctx_decode"] = bench_decode(torch, gqa, synth, "ragged_longctx_decode_bf16",
                                                          8, max(20, args.steps // 5), 3)
        secondary["llama7b_decode_G8_f16"] = bench_decode(torch, gqa, synth, name, 8, args.steps,
                                                           args.warmup, dtype="f16")
        # prefill runs the matrix cores flat out: its first ~20 calls after the
        # memory-bound decode work run ~20% slower while the clock ramps up, so
        # it gets PREFILL_WARMUP untimed calls (about 35 ms) first
        secondary["causal_prefill"] = bench_prefill(torch, gqa, synth, max(20, args.steps // 5),
                                                    PREFILL_WARMUP)
        secondary["causal_prefill_f16"] = bench_prefill(torch, gqa, synth, max(20, args.steps // 5),
                                                        PREFILL_WARMUP, dtype="f16")
        secondary["prefill_chunk_2048_after_2048"] = bench_prefill_chunk(torch, gqa, synth,
                                                                         max(20, args.steps // 5),
                                                                         PREFILL_WARMUP)
        secondary["gqkva_decode_q4_kv8"] = bench_gqkva_decode(torch, gqa, synth, args.steps, args.warmup)
        secondary["t5xxl_meanpool"] = bench_meanpool(torch, gqa, synth, args.steps, args.warmup)
        secondary["hbm_copy_probe"] = bench_copy_probe(torch, args.steps)
        secondary["hbm_read_probe"] = bench_read_probe(torch, args.steps)

    traffic = stored_traffic()
    roofline = {"bound": "hbm", "achieved": head["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(head["GBps"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "decode_mfma_kernel<128,1> (split merge fused)",
                "algorithmic_bytes_per_launch": head["bytes_per_call"]}
    line = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": head["B"], "H": head["H"], "G": G, "d": head["d"],
                   "N": head["N"], "splits": head["splits"], "replicas": head["replicas"]},
        "tokens_per_s": head["tokens_per_s"],
        "roofline": roofline,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "gcn_arch": getattr(props, "gcnArchName", "")},
        "secondary": secondary,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, synth, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
