"""GPU check of the probe library's direct-call decode timer (the benchmark's
second timing method): it calls the decode entry point it is given, rotating
over the input sets, and leaves the output of its last call."""

import ctypes
import os

import pytest
import torch

import grouped_query_decode_amd as gqa
import synth
from helpers import announce, need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_direct_call_timer_runs_the_entry_point():
    need_gpu()
    lib = gqa.load_library()
    probe = ctypes.CDLL(os.path.join(os.path.dirname(gqa.library_path()), "libgqa_probe.so"))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    f = probe.gqa_probe_time_decode_calls
    f.argtypes = ([vp] * 5 + [i32, vp] + [i32] * 5 + [ctypes.c_float] + [i32] * 2 +
                  [vp, ctypes.c_size_t, i32, i32, vp, ctypes.c_size_t, vp, vp, vp])
    f.restype = i32
    B, H, G, d, N = 4, 32, 8, 128, 600
    announce("probe direct-call timer, 3 input sets, 7 calls")
    xs = [synth.decode_inputs(B, H, G, d, N, dtype="bf16", seed=50 + r, device=DEV, seqlens="uniform",
                              nan_tail=True) for r in range(3)]
    scale = synth.scale_for(d)
    ws = torch.zeros(max(gqa.decode_workspace_bytes(B, H, G, d, N), 1), dtype=torch.uint8, device=DEV)
    out = torch.full_like(xs[0]["q"], float("nan"))
    arr = lambda key: (vp * 3)(*[x[key].data_ptr() for x in xs])  # noqa: E731
    lead = torch.ones(1 << 24, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    ms = ctypes.c_float(-1.0)
    stream = vp(torch.cuda.current_stream().cuda_stream)
    fn = ctypes.cast(lib.gqa_decode_split, vp)
    # 2 warmup calls (input sets 0, 1), then 7 timed calls (sets 0, 1, 2, 0, 1, 2, 0)
    rc = f(fn, arr("q"), arr("k_cache"), arr("v_cache"), arr("seqlens"), 3, vp(out.data_ptr()), B, H, G, d, N,
           scale, gqa.DTYPE_CODES[torch.bfloat16], 0, vp(ws.data_ptr()), ws.numel(), 2, 7,
           vp(lead.data_ptr()), lead.numel(), vp(sink.data_ptr()), stream, ctypes.byref(ms))
    torch.cuda.synchronize()
    assert rc == 0
    assert ms.value > 0.0
    # the last timed call read input set 6 % 3 = 0: its output bits are the library's
    want = gqa.decode(xs[0]["q"], xs[0]["k_cache"], xs[0]["v_cache"], xs[0]["seqlens"], scale=scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
