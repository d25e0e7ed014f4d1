"""gqa_decode_noalloc (decode with the library's static per-GPU scratch, for
callers that cannot allocate) against gqa_decode_split with a caller
workspace: same kernels, so the outputs must be bit-identical for the same
split count; both are also held to the float64 oracle's tolerance.  Two calls
in a row, the second with a smaller input (fewer sequences, fewer splits), so
the second call runs over scratch that still holds the first call's partials."""

import numpy as np
import pytest
import torch

import grouped_query_decode_amd as gqa
import oracle
import synth
from helpers import announce, assert_close, need_gpu, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    gqa.load_library()


def _oracle(x, scale):
    return oracle.decode_ref(to64(x["q"]), to64(x["k_cache"]), to64(x["v_cache"]),
                             x["seqlens"].cpu().numpy(), scale)


def _pair(x, scale, num_splits):
    """(no-alloc output, workspace output) of one decode."""
    out_na = torch.empty_like(x["q"])
    gqa.decode_noalloc(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], out_na, scale=scale,
                       num_splits=num_splits)
    ws = torch.zeros(max(gqa.decode_workspace_bytes(*x["q"].shape[:2], x["k_cache"].shape[1],
                                                    x["q"].shape[2], x["k_cache"].shape[2],
                                                    num_splits), 1),
                     dtype=torch.uint8, device=DEV)
    out_ws = gqa.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale,
                        workspace=ws, num_splits=num_splits)
    torch.cuda.synchronize()
    return out_na, out_ws


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_matches_workspace_decode_two_calls(dt):
    dtype = {"bf16": torch.bfloat16, "f32": torch.float32}[dt]
    # first call: Llama-7B-sized layer with 3 forced splits (the planner runs
    # this shape unsplit), second: a smaller ragged batch with NaN beyond the
    # lengths and more forced splits than the first call had (slots the first
    # call left are stale)
    cases = [
        dict(B=16, H=32, G=8, d=128, N=1024, seqlens="uniform", splits=3, seed=40),
        dict(B=3, H=8, G=2, d=64, N=700, seqlens=[700, 1, 333], splits=7, seed=41),
    ]
    for i, c in enumerate(cases):
        announce(f"decode_noalloc {dt} call {i}: {c}")
        x = synth.decode_inputs(c["B"], c["H"], c["G"], c["d"], c["N"], dtype=dt, seed=c["seed"],
                                device=DEV, seqlens=c["seqlens"], nan_tail=c["seqlens"] != "uniform")
        scale = synth.scale_for(c["d"])
        out_na, out_ws = _pair(x, scale, c["splits"])
        assert torch.equal(out_na.view(torch.int16 if dt == "bf16" else torch.int32),
                           out_ws.view(torch.int16 if dt == "bf16" else torch.int32)), f"call {i}"
        assert_close(out_na, _oracle(x, scale), dtype, f"noalloc call {i}")


def test_noalloc_repeated_calls_are_deterministic():
    announce("decode_noalloc bf16 repeated, G=1 (32 queries per K/V head)")
    x = synth.decode_inputs(16, 32, 1, 128, 1024, dtype="bf16", seed=42, device=DEV)
    scale = synth.scale_for(128)
    outs = []
    for _ in range(3):
        o = torch.empty_like(x["q"])
        gqa.decode_noalloc(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], o, scale=scale)
        outs.append(o)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert_close(outs[0], _oracle(x, scale), torch.bfloat16, "noalloc G=1")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    announce("decode_noalloc oversize (host-side rejection)")
    q = torch.zeros((4096, 64, 128), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((4096, 1, 1, 128), dtype=torch.bfloat16, device=DEV)
    sl = torch.ones((4096,), dtype=torch.int32, device=DEV)
    # 4096 x 64 heads x 128 with 1 position needs no split: accepted
    gqa.decode_noalloc(q, kc, kc, sl, torch.empty_like(q))
    torch.cuda.synchronize()
    kc2 = torch.zeros((64, 1, 4096, 128), dtype=torch.bfloat16, device=DEV)
    q2 = torch.zeros((64, 1024, 128), dtype=torch.bfloat16, device=DEV)
    sl2 = torch.full((64,), 4096, dtype=torch.int32, device=DEV)
    with pytest.raises(gqa.GQAError) as e:
        gqa.decode_noalloc(q2, kc2, kc2, sl2, torch.empty_like(q2), num_splits=16)
    assert e.value.status_name == "GQA_ERR_WORKSPACE"
    assert "static scratch" in str(e.value)
