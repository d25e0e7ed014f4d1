"""Host-side checks of the seeded input generators (no attention arithmetic here)."""

import numpy as np
import torch

import synth


def test_query_identical_across_group_sweep():
    qs = [synth.decode_inputs(2, 8, G, 16, 12, dtype="bf16", seed=5)["q"] for G in (8, 2, 1)]
    assert all(torch.equal(qs[0], q) for q in qs[1:])


def test_determinism_and_seed_dependence():
    a = synth.decode_inputs(2, 4, 2, 8, 10, dtype="f32", seed=1)
    b = synth.decode_inputs(2, 4, 2, 8, 10, dtype="f32", seed=1)
    c = synth.decode_inputs(2, 4, 2, 8, 10, dtype="f32", seed=2)
    for key in ("q", "k_cache", "v_cache", "seqlens"):
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["k_cache"], c["k_cache"])


def test_uniform_lengths_and_nan_tail():
    x = synth.decode_inputs(16, 4, 2, 8, 40, dtype="bf16", seed=3, seqlens="uniform", nan_tail=True)
    sl = x["seqlens"]
    assert sl.dtype == torch.int32 and int(sl.min()) >= 1 and int(sl.max()) <= 40
    for b in range(16):
        s = int(sl[b])
        for t in (x["k_cache"], x["v_cache"]):
            assert torch.isfinite(t[b, :, :s].float()).all()
            assert torch.isnan(t[b, :, s:].float()).all()


def test_explicit_lengths_and_shapes():
    x = synth.decode_inputs(3, 8, 4, 64, 20, dtype="f32", seed=0, seqlens=[0, 7, 20])
    assert x["q"].shape == (3, 8, 64) and x["k_cache"].shape == (3, 4, 20, 64)
    assert x["seqlens"].tolist() == [0, 7, 20]
    p = synth.prefill_inputs(2, 9, 8, 2, 16, dtype="bf16", seed=0)
    assert p["q"].shape == (2, 9, 8, 16) and p["k"].shape == (2, 9, 2, 16)
    w = synth.meanpool_inputs(8, (5, 3), dtype="bf16")["w"]
    assert w.shape == (8, 5, 3) and w.dtype == torch.bfloat16


def test_std_and_bf16_rounding():
    p = synth.prefill_inputs(1, 64, 4, 1, 64, dtype="f32", seed=0, std=0.5)
    p1 = synth.prefill_inputs(1, 64, 4, 1, 64, dtype="f32", seed=0, std=1.0)
    assert torch.equal(p["q"], p1["q"] * 0.5)
    b = synth.prefill_inputs(1, 64, 4, 1, 64, dtype="bf16", seed=0, std=1.0)
    assert torch.equal(b["q"], p1["q"].to(torch.bfloat16))
    x = synth.to_f64(b["q"])
    assert x.dtype == np.float64 and np.array_equal(x, b["q"].float().numpy())


def test_scale_is_float32_value():
    s = synth.scale_for(128)
    assert s == float(np.float32(s)) and abs(s - 128 ** -0.5) < 1e-8
    assert synth.scale_for(64) == 0.125


def test_workload_registry_shapes():
    w = synth.WORKLOADS
    assert w["llama7b_decode_bf16"].G_sweep == (32, 8, 4, 1)
    assert w["ragged_longctx_decode_bf16"].nan_tail
    assert w["causal_prefill_bf16"].std == 0.5
    for wl in w.values():
        if wl.kind in ("decode", "prefill"):
            assert wl.H % wl.G == 0
