"""GPU parity of gqa_prefill_causal and kv_meanpool_heads against the float64 oracle."""

import numpy as np
import pytest
import torch

import grouped_query_decode_amd as gqa
import oracle
import synth
from helpers import announce, assert_close, bf16_ulp_distance, f32_attention_bound, need_gpu, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    gqa.load_library()


def _prefill(x, scale):
    o = gqa.prefill_causal(x["q"], x["k"], x["v"], scale=scale)
    torch.cuda.synchronize()
    return o


PREFILL_CASES = [
    # B, T, H, G, d, dtype
    (2, 200, 8, 2, 128, "bf16"),
    (1, 333, 32, 8, 128, "bf16"),
    (2, 130, 8, 8, 64, "bf16"),      # n_rep = 1
    (2, 97, 8, 4, 64, "bf16"),       # n_rep = 2
    (2, 150, 16, 4, 64, "bf16"),     # n_rep = 4 at d = 64 (4 heads per workgroup)
    (1, 200, 32, 4, 64, "bf16"),     # n_rep = 8 at d = 64
    (1, 150, 32, 1, 128, "bf16"),    # n_rep = 32
    (1, 64, 24, 8, 128, "bf16"),     # n_rep = 3: one padded head quad
    (2, 150, 20, 4, 128, "bf16"),    # n_rep = 5: second quad has 3 padding slots
    (1, 200, 48, 8, 64, "bf16"),     # n_rep = 6 at d = 64
    (1, 120, 28, 4, 128, "f16"),     # n_rep = 7
    (1, 1, 8, 2, 128, "bf16"),       # single position
    (2, 100, 8, 2, 64, "f32"),
    (1, 70, 16, 16, 128, "f32"),
]


@pytest.mark.parametrize("B,T,H,G,d,dt", PREFILL_CASES)
def test_prefill_cases(B, T, H, G, d, dt):
    announce(f"prefill B={B} T={T} H={H} G={G} d={d} {dt}")
    x = synth.prefill_inputs(B, T, H, G, d, dtype=dt, seed=T + H, device=DEV, std=0.5)
    scale = synth.scale_for(d)
    out = _prefill(x, scale)
    ref = oracle.prefill_causal_ref(to64(x["q"]), to64(x["k"]), to64(x["v"]), scale)
    assert_close(out, ref, x["q"].dtype, "prefill")
    # row 0 attends only key 0: exactly its value
    want0 = x["v"][:, 0].repeat_interleave(H // G, dim=1)
    assert torch.equal(out[:, 0], want0)


def _ramp_inputs(B, T, H, G, d, dt, step_log2, seed, spike=None):
    """Seeded prefill inputs whose scores drift by step_log2 (base 2) every 64 keys.

    Dimension 0 of every query is a constant a and dimension 0 of key j grows
    linearly with j, so scale*log2(e)*q.k[j] = step_log2*j/64 + noise: a
    positive step raises each row's maximum tile after tile (above 8 per tile
    the kernel must rescale its running output every tile), a negative one
    keeps the maximum at key 0.  With spike=(position, jump) that key alone gets
    an extra score of jump (base 2).
    """
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn(B, T, H, d, generator=gen) * 0.5
    k = torch.randn(B, T, G, d, generator=gen) * 0.5
    v = torch.randn(B, T, G, d, generator=gen)
    a = 4.0
    c = synth.scale_for(d) * 1.4426950408889634 * a          # base-2 score per unit of k[..., 0]
    q[..., 0] = a
    k[..., 0] = (step_log2 / 64.0) * torch.arange(T, dtype=torch.float32)[None, :, None] / c
    if spike is not None:
        pos, jump = spike
        k[:, pos, :, 0] += jump / c
    dtype = synth.torch_dtype(dt)
    return {n: t.to(dtype).to(DEV) for n, t in (("q", q), ("k", k), ("v", v))}


@pytest.mark.parametrize("step", [-12.0, 4.0, 9.0, 12.0])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_prefill_growing_row_maxima(step, dt):
    """Row maxima that keep growing tile after tile (and one that never grows):
    the running output is rescaled on exactly those tiles, and the result must
    not depend on when that happens."""
    announce(f"prefill ramp step={step} {dt}")
    B, T, H, G, d = 1, 520, 8, 2, 128
    x = _ramp_inputs(B, T, H, G, d, dt, step, seed=int(step * 10) + 7)
    scale = synth.scale_for(d)
    out = _prefill(x, scale)
    ref = oracle.prefill_causal_ref(to64(x["q"]), to64(x["k"]), to64(x["v"]), scale)
    assert_close(out, ref, x["q"].dtype, f"prefill ramp {step}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_prefill_late_score_spike(dt):
    """One key far into the prompt outscores everything before it by 2^40:
    rows at or after it must switch to it (their running output is rescaled by
    about 2^-40), rows before it must not see it."""
    announce(f"prefill late spike {dt}")
    B, T, H, G, d = 2, 400, 8, 2, 128
    x = _ramp_inputs(B, T, H, G, d, dt, 0.0, seed=11, spike=(301, 40.0))
    scale = synth.scale_for(d)
    out = _prefill(x, scale)
    ref = oracle.prefill_causal_ref(to64(x["q"]), to64(x["k"]), to64(x["v"]), scale)
    assert_close(out, ref, x["q"].dtype, "prefill spike")


def test_prefill_chunk_growing_row_maxima():
    """The chunked form (queries after a cached prefix) on growing maxima."""
    announce("prefill_chunk ramp")
    B, T, H, G, d, ctx = 1, 200, 8, 2, 128, 300
    x = _ramp_inputs(B, ctx + T, H, G, d, "bf16", 10.0, seed=5)
    scale = synth.scale_for(d)
    kc = x["k"].transpose(1, 2).contiguous()                 # [B, G, Nmax, d] cache layout
    vc = x["v"].transpose(1, 2).contiguous()
    q = x["q"][:, ctx:].contiguous()
    cl = torch.full((B,), ctx, dtype=torch.int32, device=DEV)
    out = gqa.prefill_chunk(q, kc, vc, cl, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.prefill_chunk_ref(to64(q), to64(kc), to64(vc), cl.cpu().numpy(), scale)
    assert_close(out, ref, q.dtype, "prefill_chunk ramp")


def test_prefill_row_matches_decode():
    """Prefill row i equals a decode step over the first i+1 positions."""
    announce("prefill vs decode rows")
    B, T, H, G, d = 2, 300, 32, 8, 128
    x = synth.prefill_inputs(B, T, H, G, d, dtype="bf16", seed=3, device=DEV)
    scale = synth.scale_for(d)
    out = _prefill(x, scale)
    kc = x["k"].transpose(1, 2).contiguous()
    vc = x["v"].transpose(1, 2).contiguous()
    for i in (0, 1, 63, 64, 65, 127, 128, 299):
        dec = gqa.decode(x["q"][:, i].contiguous(), kc, vc,
                         torch.full((B,), i + 1, dtype=torch.int32, device=DEV), scale=scale)
        torch.cuda.synchronize()
        diff = (out[:, i].float() - dec.float()).abs().max().item()
        assert diff <= 1.6e-2, (i, diff)


def test_prefill_deterministic():
    """Repeated calls give identical bits (with other allocations in between, so
    that a workgroup reading an LDS tile another wave already replaced would
    show up as a changed row block)."""
    announce("prefill determinism")
    x = synth.prefill_inputs(1, 512, 32, 8, 128, dtype="bf16", seed=4, device=DEV)
    a = _prefill(x, 0.09).clone()
    for _ in range(12):
        junk = torch.randn(1 << 22, device=DEV)
        b = _prefill(x, 0.09)
        assert torch.equal(a, b)
        del junk


def test_causal_prefill_full_size_every_row():
    """The 4096-token prompt workload at full size (B=2, H=32, G=8, d=128):
    every row of every (sequence, head) against the oracle, plus the error
    statistics in units of the output's ulp."""
    w = synth.WORKLOADS["causal_prefill_bf16"]
    announce("prefill full size B=2 T=4096 H=32 G=8 d=128, every row")
    x = synth.prefill_inputs(w.B, w.N, w.H, w.G, w.d, dtype="bf16", seed=w.seed, device=DEV,
                             std=w.std)
    scale = synth.scale_for(w.d)
    out = _prefill(x, scale)
    assert torch.isfinite(out.float()).all()
    ref = oracle.prefill_causal_ref(x["q"].double().cpu().numpy(), x["k"].double().cpu().numpy(),
                                    x["v"].double().cpu().numpy(), scale)
    stats = assert_close(out, ref, torch.bfloat16, "prefill full, every row")
    ulps = bf16_ulp_distance(out, ref)
    print(f"prefill full size, all {w.B * w.N} rows x {w.H} heads: {stats}; "
          f"outputs equal to RNE(oracle): {float((ulps == 0).mean()):.4f}, within 1 ulp: "
          f"{float((ulps <= 1).mean()):.6f}")


# ---------------------------------------------------------------------------
# kv_meanpool_heads
# ---------------------------------------------------------------------------

def _meanpool(w, G):
    o = gqa.meanpool_heads(w, G)
    torch.cuda.synchronize()
    return o


def test_meanpool_t5xxl_projection_bf16():
    wl = synth.WORKLOADS["t5xxl_meanpool_bf16"]
    announce("meanpool [64,4096,64] -> 8 bf16")
    for seed in (0, 1):          # one call for the K weights, one for the V weights
        w = synth.meanpool_inputs(wl.H, wl.per_head_shape, dtype="bf16", seed=seed, device=DEV)["w"]
        out = _meanpool(w, wl.G)
        ref = oracle.meanpool_ref(to64(w), wl.G)
        ulps = bf16_ulp_distance(out, ref)
        assert ulps.max() <= 1, ulps.max()
        exact = float((ulps == 0).mean())
        assert exact >= 0.99, exact


@pytest.mark.parametrize("H,G,shape,dt", [
    (8, 2, (16, 64), "f32"), (8, 8, (5, 3), "bf16"), (6, 3, (7, 5), "bf16"),
    (6, 1, (33,), "f32"), (64, 8, (4096, 64), "f32"), (32, 4, (13, 8), "bf16"),
])
def test_meanpool_cases(H, G, shape, dt):
    announce(f"meanpool H={H} G={G} shape={shape} {dt}")
    w = synth.meanpool_inputs(H, shape, dtype=dt, seed=H + G, device=DEV)["w"]
    out = _meanpool(w, G)
    ref = oracle.meanpool_ref(to64(w), G)
    if dt == "f32":
        assert np.abs(to64(out) - ref).max() <= 1e-5
    else:
        assert bf16_ulp_distance(out, ref).max() <= 1
    if G == H:
        assert torch.equal(out, w)


@pytest.mark.parametrize("count,H,G,shape,dt", [
    (2, 64, 8, (4096, 64), "bf16"),          # one T5-XXL layer's K and V projections
    (16, 8, 2, (16, 64), "f32"),             # a full batch
    (17, 6, 3, (7, 5), "bf16"),              # one batch of 16 and one of 1; odd size (scalar kernel)
    (3, 32, 4, (13, 8), "f16"),
    (1, 8, 8, (5, 3), "bf16"),
])
def test_meanpool_batch_matches_single_calls(count, H, G, shape, dt):
    """kv_meanpool_heads_batch: every projection bit-identical to its own
    kv_meanpool_heads call, and within the single call's bound of the oracle."""
    announce(f"meanpool batch count={count} H={H} G={G} shape={shape} {dt}")
    ws = [synth.meanpool_inputs(H, shape, dtype=dt, seed=100 + j, device=DEV)["w"] for j in range(count)]
    outs = gqa.meanpool_heads_batch(ws, G)
    torch.cuda.synchronize()
    assert len(outs) == count
    for w, out in zip(ws, outs):
        single = _meanpool(w, G)
        assert torch.equal(out.view(torch.uint8), single.view(torch.uint8))
        ref = oracle.meanpool_ref(to64(w), G)
        if dt == "f32":
            assert np.abs(to64(out) - ref).max() <= 1e-5
        elif dt == "bf16":
            assert bf16_ulp_distance(out, ref).max() <= 1
        else:   # within one fp16 ulp of the oracle rounded to nearest even
            got = out.cpu().numpy().view(np.int16).astype(np.int64)
            want = ref.astype(np.float16).view(np.int16).astype(np.int64)
            assert np.abs(got - want).max() <= 1


def test_meanpool_identical_heads_bit_exact():
    announce("meanpool identical heads")
    base = synth.meanpool_inputs(1, (512, 64), dtype="bf16", seed=3, device=DEV)["w"]
    w = base.expand(16, 512, 64).contiguous()
    out = _meanpool(w, 4)
    assert torch.equal(out, base.expand(4, 512, 64))


def _random_prefill_shapes(n, seed):
    """A fixed list of shapes drawn once from a seeded generator: both head
    sizes, every group size the matrix-core kernel takes plus ones it hands to
    the vector kernel, all three dtypes, prompt lengths across tile edges."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        n_rep = int(rng.choice([1, 2, 3, 4, 8, 12]))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 3))
        T = int(rng.integers(1, 260))
        dt = str(rng.choice(["bf16", "f16", "f32"]))
        shapes.append((B, T, G * n_rep, G, d, dt))
    return shapes


@pytest.mark.parametrize("case", _random_prefill_shapes(16, 77))
def test_prefill_random_shapes(case):
    B, T, H, G, d, dt = case
    announce(f"prefill random B={B} T={T} H={H} G={G} d={d} {dt}")
    x = synth.prefill_inputs(B, T, H, G, d, dtype=dt, seed=T + 3 * H + d, device=DEV, std=0.5)
    scale = synth.scale_for(d)
    out = _prefill(x, scale)
    ref = oracle.prefill_causal_ref(to64(x["q"]), to64(x["k"]), to64(x["v"]), scale)
    assert_close(out, ref, x["q"].dtype, f"prefill random {case}")


# float32 at scale 2: held to float32's own forward-error bound
# (f32_attention_bound) rather than the fixed float32 bound set for 1/sqrt(d)
@pytest.mark.parametrize("scale,dt", [(0.0, "bf16"), (-0.3, "bf16"), (2.0, "bf16"),
                                      (0.0, "f32"), (-0.3, "f32"), (2.0, "f32")])
def test_prefill_unusual_scales(scale, dt):
    """As for decode: the mean of the visible rows at scale 0, the least similar
    keys favoured at a negative scale, a nearly hard softmax at scale 2."""
    announce(f"prefill scale={scale} {dt}")
    x = synth.prefill_inputs(1, 300, 8, 2, 128, dtype=dt, seed=19, device=DEV, std=1.0)
    out = _prefill(x, scale)
    ref = oracle.prefill_causal_ref(to64(x["q"]), to64(x["k"]), to64(x["v"]), scale)
    if dt == "f32" and scale == 2.0:
        q, k, v = to64(x["q"])[0], to64(x["k"])[0], to64(x["v"])[0]     # [T, H, d], [T, G, d]
        T, H = q.shape[0], q.shape[1]
        n_rep = H // k.shape[1]
        causal = np.tril(np.ones((T, T), dtype=bool))
        o64 = to64(out)[0]
        worst = 0.0
        for h in range(H):
            exact, tol = f32_attention_bound(q[:, h], k[:, h // n_rep], v[:, h // n_rep], scale, causal)
            np.testing.assert_allclose(exact, ref[0, :, h], rtol=1e-11, atol=1e-12)
            err = np.abs(o64[:, h] - ref[0, :, h])
            assert (err <= tol).all(), (h, float((err / tol).max()))
            worst = max(worst, float((err / tol).max()))
        print(f"prefill f32 scale 2: largest error / bound = {worst:.3g}")
        return
    assert_close(out, ref, x["q"].dtype, f"prefill scale={scale}")
