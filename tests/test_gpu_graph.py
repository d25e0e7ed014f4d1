"""The library's calls captured into a HIP graph and replayed: every replay must
give the same bits as the eager calls.  The benchmark times the kernels this
way, and a graph replays whatever the kernels leave behind (the split-arrival
counters each decode resets for the next call, stale split partials), so each
replay is checked, with eager work and synchronisations between replays and
the outputs poisoned with NaN before each one.  Workspaces are allocated and
zero-filled before capture, as a caller under capture must."""

import pytest
import torch

import grouped_query_decode_amd as gqa
import synth
from helpers import announce, need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    gqa.load_library()


def _check_replays(calls, outs, what):
    """calls: closures that together write every tensor of outs."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        # eager work between replays: the same calls outside the graph, into scratch outputs
        calls[r % len(calls)]()
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"{what}: replay {r}, output {i}"
    del graph


def _decode_calls(cases, dt, noalloc=False):
    calls, outs = [], []
    for c in cases:
        x = synth.decode_inputs(c["B"], c["H"], c["G"], c["d"], c["N"], dtype=dt, seed=c["seed"],
                                device=DEV, seqlens=c["seqlens"], nan_tail=c["seqlens"] != "full")
        out = torch.empty_like(x["q"])
        scale = synth.scale_for(c["d"])
        if noalloc:
            calls.append(lambda x=x, out=out, c=c, scale=scale: gqa.decode_noalloc(
                x["q"], x["k_cache"], x["v_cache"], x["seqlens"], out, scale=scale,
                num_splits=c["splits"]))
        else:
            ws = torch.zeros(max(gqa.decode_workspace_bytes(c["B"], c["H"], c["G"], c["d"], c["N"],
                                                            c["splits"]), 1),
                             dtype=torch.uint8, device=DEV)
            calls.append(lambda x=x, out=out, c=c, ws=ws, scale=scale: gqa.decode(
                x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale, out=out, workspace=ws,
                num_splits=c["splits"]))
        outs.append(out)
    return calls, outs


# three calls per graph, each with its own inputs, workspace and output
DECODE_CASES = [
    dict(B=4, H=32, G=8, d=128, N=1024, seqlens="full", splits=0, seed=301),      # planned splits, in-kernel merge
    dict(B=3, H=8, G=2, d=64, N=700, seqlens=[700, 1, 333], splits=7, seed=302),   # ragged, NaN past the lengths
    dict(B=2, H=32, G=1, d=128, N=512, seqlens=[512, 77], splits=0, seed=303),     # 32 queries per K/V head
]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_decode_graph_replays_match_eager(dt):
    # f32 runs the vector-unit kernel and the separate merge kernel
    announce(f"decode graph replay {dt}")
    calls, outs = _decode_calls(DECODE_CASES, dt)
    _check_replays(calls, outs, f"decode {dt}")


def test_decode_noalloc_graph_replays_match_eager():
    announce("decode_noalloc graph replay bf16")
    calls, outs = _decode_calls(DECODE_CASES, "bf16", noalloc=True)
    calls[0]()                      # the static scratch is set up outside the capture
    torch.cuda.synchronize()
    _check_replays(calls, outs, "decode_noalloc")


def test_prefill_graph_replays_match_eager():
    announce("prefill graph replay bf16 / f32")
    calls, outs = [], []
    for (B, T, H, G, d, dt, seed) in [(1, 300, 8, 2, 128, "bf16", 311), (2, 130, 4, 4, 64, "bf16", 312),
                                      (1, 70, 4, 2, 64, "f32", 313)]:
        x = synth.prefill_inputs(B, T, H, G, d, dtype=dt, seed=seed, device=DEV)
        out = torch.empty_like(x["q"])
        calls.append(lambda x=x, out=out, d=d: gqa.prefill_causal(x["q"], x["k"], x["v"],
                                                                  scale=synth.scale_for(d), out=out))
        outs.append(out)
    _check_replays(calls, outs, "prefill")


def test_meanpool_graph_replays_match_eager():
    announce("meanpool graph replay bf16")
    ws = [synth.meanpool_inputs(64, (256, 64), dtype="bf16", seed=320 + i, device=DEV)["w"] for i in range(3)]
    outs = [torch.empty((8, 256, 64), dtype=torch.bfloat16, device=DEV) for _ in ws[:2]]
    single = torch.empty((8, 256, 64), dtype=torch.bfloat16, device=DEV)
    calls = [lambda: gqa.meanpool_heads_batch(ws[:2], 8, outs[:2]),
             lambda: gqa.meanpool_heads(ws[2], 8, single)]
    _check_replays(calls, outs[:2] + [single], "meanpool")
