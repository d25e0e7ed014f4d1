"""GPU parity of gqa_decode against the float64 oracle (through the C ABI binding)."""

import numpy as np
import pytest
import torch

import grouped_query_decode_amd as gqa
import oracle
import synth
from helpers import announce, assert_close, f32_attention_bound, need_gpu, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    gqa.load_library()


def _run(x, scale, num_splits=0, out=None):
    o = gqa.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale, out=out,
                   num_splits=num_splits)
    torch.cuda.synchronize()
    return o


def _oracle(x, scale, rows=None):
    sl = x["seqlens"].cpu().numpy()
    if rows is None:
        return oracle.decode_ref(to64(x["q"]), to64(x["k_cache"]), to64(x["v_cache"]), sl, scale)
    # only the listed sequences, copying just their attended cache rows
    outs = []
    for b in rows:
        n = oracle.attended_length(sl[b], x["k_cache"].shape[2])
        n = max(n, 1)
        q = to64(x["q"][b:b + 1])
        k = to64(x["k_cache"][b:b + 1, :, :n])
        v = to64(x["v_cache"][b:b + 1, :, :n])
        outs.append(oracle.decode_ref(q, k, v, [sl[b]], scale)[0])
    return np.stack(outs)


# ---------------------------------------------------------------------------
# the tiny float32 workload: 8 heads, G = 2 (GQA), 8 (MHA), 1 (MQA)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G", [2, 8, 1])
def test_tiny_f32_group_sweep(G):
    w = synth.WORKLOADS["tiny_decode_f32"]
    announce(f"decode tiny f32 G={G}")
    x = synth.decode_inputs(w.B, w.H, G, w.d, w.N, dtype="f32", seed=w.seed, device=DEV)
    scale = synth.scale_for(w.d)
    assert_close(_run(x, scale), _oracle(x, scale), torch.float32, f"tiny G={G}")


def test_tiny_f32_repeat_kv_reproduces_gqa():
    announce("decode tiny f32 repeat_kv")
    x = synth.decode_inputs(1, 8, 2, 64, 128, dtype="f32", seed=0, device=DEV)
    scale = synth.scale_for(64)
    a = _run(x, scale)
    xr = dict(x)
    xr["k_cache"] = x["k_cache"].repeat_interleave(4, dim=1).contiguous()
    xr["v_cache"] = x["v_cache"].repeat_interleave(4, dim=1).contiguous()
    b = _run(xr, scale)
    assert (a - b).abs().max().item() <= 1e-6


# ---------------------------------------------------------------------------
# shapes that span several tiles, ragged tails, every group size
# ---------------------------------------------------------------------------

CASES = [
    # B, H, G, d, Nmax, dtype
    (3, 8, 2, 64, 300, "bf16"),
    (2, 32, 8, 128, 777, "bf16"),
    (2, 32, 32, 128, 129, "bf16"),
    (2, 32, 1, 128, 200, "bf16"),
    (2, 64, 8, 64, 450, "bf16"),
    (2, 16, 16, 64, 97, "bf16"),
    (2, 32, 2, 128, 160, "bf16"),
    (2, 64, 2, 64, 130, "bf16"),      # n_rep = 32: two work groups of 16 per K/V head
    (2, 64, 1, 128, 333, "bf16"),     # n_rep = 64: four work groups of 16 per K/V head
    (2, 48, 1, 64, 150, "f16"),       # n_rep = 48: three work groups of 16
    (2, 40, 2, 128, 90, "bf16"),      # n_rep = 20: one work group, two tiles of heads
    (2, 24, 8, 128, 140, "bf16"),     # n_rep = 3
    (3, 8, 2, 128, 300, "f32"),
    (2, 32, 4, 64, 260, "f32"),
    (2, 32, 1, 64, 100, "f32"),       # n_rep = 32 on the vector units
]


@pytest.mark.parametrize("B,H,G,d,n_max,dt", CASES)
def test_decode_ragged_cases(B, H, G, d, n_max, dt):
    announce(f"decode B={B} H={H} G={G} d={d} Nmax={n_max} {dt}")
    rng = np.random.default_rng(B * 1000 + H + G + d + n_max)
    lens = [int(rng.integers(1, n_max + 1)) for _ in range(B)]
    lens[0] = n_max
    if B > 2:
        lens[2] = 1
    x = synth.decode_inputs(B, H, G, d, n_max, dtype=dt, seed=7, device=DEV, seqlens=lens,
                            nan_tail=True)
    scale = synth.scale_for(d)
    assert_close(_run(x, scale), _oracle(x, scale), x["q"].dtype, "ragged")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("S", [1, 2, 7, 64, 1000])
def test_forced_split_counts(dt, S):
    announce(f"decode forced splits S={S} {dt}")
    x = synth.decode_inputs(3, 16, 4, 128, 1000, dtype=dt, seed=3, device=DEV,
                            seqlens=[1000, 513, 31], nan_tail=True)
    scale = synth.scale_for(128)
    assert_close(_run(x, scale, num_splits=S), _oracle(x, scale), x["q"].dtype, f"S={S}")


@pytest.mark.parametrize("S", [1, 3, 7, 64])
def test_forced_split_counts_large_group(S):
    """n_rep = 32 (run as two work groups of 16 per K/V head) with every split count."""
    announce(f"decode n_rep=32 forced splits S={S}")
    x = synth.decode_inputs(3, 32, 1, 128, 1000, dtype="bf16", seed=13, device=DEV,
                            seqlens=[1000, 1, 517], nan_tail=True)
    scale = synth.scale_for(128)
    assert_close(_run(x, scale, num_splits=S), _oracle(x, scale), x["q"].dtype, f"n_rep=32 S={S}")


def test_lengths_zero_and_beyond_capacity():
    announce("decode seqlen 0 and > Nmax")
    x = synth.decode_inputs(4, 8, 2, 64, 96, dtype="bf16", seed=4, device=DEV,
                            seqlens=[0, 96, 500, -3])
    scale = 0.125
    out = _run(x, scale).clone()
    ref = _oracle(x, scale)
    assert torch.equal(out[0], torch.zeros_like(out[0]))
    assert torch.equal(out[3], torch.zeros_like(out[3]))
    assert_close(out, ref, torch.bfloat16, "lengths")
    # a length of 500 behaves exactly like the capacity 96
    x2 = dict(x)
    x2["seqlens"] = torch.tensor([0, 96, 96, 0], dtype=torch.int32, device=DEV)
    out2 = _run(x2, scale)
    assert torch.equal(out, out2)


def test_empty_cache_capacity_gives_zeros():
    announce("decode Nmax = 0")
    q = torch.randn(2, 8, 64, device=DEV).to(torch.bfloat16)
    k = torch.empty(2, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    out = torch.full_like(q, 3.0)
    gqa.decode(q, k, k, torch.tensor([0, 5], dtype=torch.int32, device=DEV), out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))


# ---------------------------------------------------------------------------
# bit-exact properties
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_masking_is_bit_exact(dt):
    """Cache rows at or beyond the length cannot change a single output bit."""
    announce(f"decode masking bits {dt}")
    B, H, G, d, n_max = 4, 32, 8, 128, 700
    lens = [700, 333, 64, 1]
    base = synth.decode_inputs(B, H, G, d, n_max, dtype=dt, seed=11, device=DEV, seqlens=lens)
    scale = synth.scale_for(d)
    outs = []
    for fill in ("nan", "random", "dominant"):
        x = {k: v.clone() for k, v in base.items()}
        for b, n in enumerate(lens):
            if fill == "nan":
                x["k_cache"][b, :, n:] = float("nan")
                x["v_cache"][b, :, n:] = float("nan")
            elif fill == "random":
                x["k_cache"][b, :, n:] = torch.randn_like(x["k_cache"][b, :, n:].float()).to(x["k_cache"].dtype)
                x["v_cache"][b, :, n:] = 1e4
            else:
                if n < n_max:
                    qg = x["q"][b].float().view(G, H // G, d).sum(1)
                    x["k_cache"][b, :, n] = (qg * 100).to(x["k_cache"].dtype)
                    x["v_cache"][b, :, n] = 1e4
        outs.append(_run(x, scale).clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    # the last attended position does count: a dominant key there takes over
    x = {k: v.clone() for k, v in base.items()}
    for b, n in enumerate(lens):
        qg = x["q"][b].float().view(G, H // G, d).sum(1)
        x["k_cache"][b, :, n - 1] = (qg * 100).to(x["k_cache"].dtype)
        x["v_cache"][b, :, n - 1] = 2.0
    out = _run(x, scale)
    assert torch.equal(out, torch.full_like(out, 2.0))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("H,G", [(32, 8), (8, 2), (64, 64), (32, 1), (24, 8)])
def test_group_map_is_bit_exact(dt, H, G):
    """V of K/V head g is a distinct power of two: every output element names its group.

    bfloat16 outputs equal the constant exactly; float32 outputs carry the
    normaliser's rounding, so there the nearest constant must be the right one.
    """
    announce(f"decode group map H={H} G={G} {dt}")
    B, d, n_max = 2, 64 if H == 64 else 128, 200
    x = synth.decode_inputs(B, H, G, d, n_max, dtype=dt, seed=5, device=DEV, seqlens=[200, 77])
    for perm in (list(range(G)), list(reversed(range(G)))):
        consts = torch.tensor([2.0 ** (gg - G // 2) for gg in perm], dtype=torch.float64)
        x["v_cache"] = consts.view(1, G, 1, 1).expand(B, G, n_max, d).to(DEV).to(x["k_cache"].dtype).contiguous()
        out = _run(x, synth.scale_for(d)).double().cpu()
        want_g = torch.tensor([oracle.kv_group_of_head(h, H, G) for h in range(H)])
        want = consts[want_g].view(1, H, 1).expand(B, H, d)
        if dt == "bf16":
            assert torch.equal(out, want)
        else:
            nearest = (out[..., None].log2() - consts.log2().view(1, 1, 1, G)).abs().argmin(-1)
            assert torch.equal(nearest, want_g.view(1, H, 1).expand(B, H, d))
            assert ((out - want).abs() / want).max().item() <= 1e-6


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_single_key_returns_its_value(dt):
    announce(f"decode single key {dt}")
    B, H, G, d = 3, 32, 8, 128
    x = synth.decode_inputs(B, H, G, d, 64, dtype=dt, seed=6, device=DEV, seqlens=[1, 1, 1])
    x["q"] = (x["q"].float() * 30).to(x["q"].dtype)
    out = _run(x, synth.scale_for(d))
    want = x["v_cache"][:, :, 0].repeat_interleave(H // G, dim=1)
    assert torch.equal(out, want)


def test_constant_values_are_exact_bf16():
    announce("decode constant V bf16")
    B, H, G, d, n = 2, 32, 4, 128, 999
    x = synth.decode_inputs(B, H, G, d, n, dtype="bf16", seed=8, device=DEV)
    x["v_cache"] = torch.full_like(x["v_cache"], 0.375)
    out = _run(x, synth.scale_for(d))
    assert torch.equal(out, torch.full_like(out, 0.375))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_deterministic(dt):
    announce(f"decode determinism {dt}")
    x = synth.decode_inputs(8, 32, 8, 128, 3000, dtype=dt, seed=9, device=DEV, seqlens="uniform")
    a = _run(x, 0.1).clone()
    b = _run(x, 0.1)
    assert torch.equal(a, b)


def test_output_guard_untouched():
    announce("decode guard canaries")
    B, H, G, d, n = 2, 32, 8, 128, 1024
    x = synth.decode_inputs(B, H, G, d, n, dtype="bf16", seed=10, device=DEV)
    pad = 4096
    buf = torch.full((pad + B * H * d + pad,), 7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[pad:pad + B * H * d].view(B, H, d)
    _run(x, synth.scale_for(d), out=out)
    assert torch.equal(buf[:pad], torch.full((pad,), 7.0, dtype=torch.bfloat16, device=DEV))
    assert torch.equal(buf[-pad:], torch.full((pad,), 7.0, dtype=torch.bfloat16, device=DEV))
    assert_close(out, _oracle(x, synth.scale_for(d)), torch.bfloat16, "guard")


# ---------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G", [32, 8, 4, 1])
def test_llama7b_decode_group_sweep(G):
    w = synth.WORKLOADS["llama7b_decode_bf16"]
    announce(f"decode llama7b G={G}")
    x = synth.decode_inputs(w.B, w.H, G, w.d, w.N, dtype="bf16", seed=w.seed, device=DEV)
    scale = synth.scale_for(w.d)
    assert_close(_run(x, scale), _oracle(x, scale), torch.bfloat16, f"llama7b G={G}")


def test_t5xxl_cross_attention_decode():
    w = synth.WORKLOADS["t5xxl_cross_decode_bf16"]
    announce("decode t5xxl cross")
    x = synth.decode_inputs(w.B, w.H, w.G, w.d, w.N, dtype="bf16", seed=w.seed, device=DEV)
    scale = synth.scale_for(w.d)
    assert_close(_run(x, scale), _oracle(x, scale), torch.bfloat16, "t5xxl")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_grid_of_many_workgroup_rounds(dt, num_splits):
    """A d = 128 grid of 1024 or more workgroups (128 sequences x 8 K/V heads;
    with 3 splits 3072), which the library launches one workgroup per compute
    unit: ragged lengths with NaN beyond them, every output row against the
    oracle."""
    B, H, G, d, n_max = 128, 32, 8, 128, 520
    announce(f"decode {B}x{H}/{G} d={d} N={n_max} {dt} splits={num_splits}")
    x = synth.decode_inputs(B, H, G, d, n_max, dtype=dt, seed=31, device=DEV, seqlens="uniform",
                            nan_tail=True)
    scale = synth.scale_for(d)
    out = _run(x, scale, num_splits=num_splits)
    assert_close(out, _oracle(x, scale), synth.torch_dtype(dt), f"{B}x{G} grid, {dt}, S={num_splits}")


def test_append_grid_of_many_workgroup_rounds():
    """The fused append on the same 1024-workgroup d = 128 grid: the new rows
    land in the caches bit for bit and the output matches the oracle."""
    B, H, G, d, n_max = 128, 32, 8, 128, 520
    announce(f"decode_append {B}x{H}/{G} d={d} N={n_max}")
    x = synth.decode_append_inputs(B, H, G, d, n_max, seed=32, device=DEV, seqlens="uniform",
                                   nan_tail=True)
    scale = synth.scale_for(d)
    k, v = x["k_cache"].clone(), x["v_cache"].clone()
    out = gqa.decode_append(x["q"], x["k_new"], x["v_new"], k, v, x["seqlens"], scale=scale)
    torch.cuda.synchronize()
    ref, k_ref, v_ref = oracle.decode_append_ref(to64(x["q"]), to64(x["k_new"]), to64(x["v_new"]),
                                                 to64(x["k_cache"]), to64(x["v_cache"]),
                                                 x["seqlens"].cpu().numpy(), scale)
    sl = x["seqlens"].cpu().numpy()
    kk, vv = to64(k), to64(v)
    for b in range(B):
        pos = oracle.append_position(sl[b], n_max)
        assert np.array_equal(kk[b, :, pos], k_ref[b, :, pos]), b
        assert np.array_equal(vv[b, :, pos], v_ref[b, :, pos]), b
    assert_close(out, ref, torch.bfloat16, "append, 1024-workgroup grid")


def _slice64(t):
    """Exact float64 host copy of a (bf16 or f32) device slice (upcast on the GPU)."""
    return t.double().cpu().numpy()


def _oracle_all_sequences(x, scale):
    """The oracle for every sequence, one sequence's attended cache rows at a time."""
    sl = x["seqlens"].cpu().numpy()
    n_max = x["k_cache"].shape[2]
    outs = []
    for b in range(x["q"].shape[0]):
        n = max(oracle.attended_length(sl[b], n_max), 1)
        outs.append(oracle.decode_ref(_slice64(x["q"][b:b + 1]), _slice64(x["k_cache"][b:b + 1, :, :n]),
                                      _slice64(x["v_cache"][b:b + 1, :, :n]), [sl[b]], scale)[0])
    return np.stack(outs)


def test_ragged_long_context_decode_all_sequences():
    """The ragged 32k workload at full size (B=64, H=32, G=8, d=128, lengths
    uniform in [1, 32768], NaN beyond each length): every output row against
    the oracle."""
    w = synth.WORKLOADS["ragged_longctx_decode_bf16"]
    announce("decode ragged long context (8 GiB cache), all 64 sequences")
    x = synth.decode_inputs(w.B, w.H, w.G, w.d, w.N, dtype="bf16", seed=w.seed, device=DEV,
                            seqlens="uniform", nan_tail=True)
    scale = synth.scale_for(w.d)
    out = _run(x, scale)
    assert torch.isfinite(out.float()).all()
    stats = assert_close(out, _oracle_all_sequences(x, scale), torch.bfloat16, "ragged long, all rows")
    print(f"ragged long context, all {w.B} sequences: {stats}")
    del x
    torch.cuda.empty_cache()


def test_ragged_long_context_masking_is_bit_exact():
    """At the ragged 32k workload's full size: the cache beyond each length
    filled with NaN, then refilled in place with random values (and huge V),
    then with a key at the first position past the length that would dominate
    every score: the output bits must not change.  A dominant key at the last
    attended position must take over (the length is not off by one)."""
    w = synth.WORKLOADS["ragged_longctx_decode_bf16"]
    announce("decode ragged long context masking bits (8 GiB cache)")
    x = synth.decode_inputs(w.B, w.H, w.G, w.d, w.N, dtype="bf16", seed=w.seed, device=DEV,
                            seqlens="uniform", nan_tail=True)
    scale = synth.scale_for(w.d)
    B, H, G, d, n_max = w.B, w.H, w.G, w.d, w.N
    lens = x["seqlens"].cpu().tolist()
    out_nan = _run(x, scale).clone()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(123)
    for b, n in enumerate(lens):
        if n < n_max:
            tail = x["k_cache"][b, :, n:]
            tail.copy_(torch.randn(tail.shape, generator=gen, device=DEV).to(tail.dtype))
            x["v_cache"][b, :, n:] = 1e4
    out_rand = _run(x, scale).clone()
    for b, n in enumerate(lens):
        if n < n_max:
            qg = x["q"][b].float().view(G, H // G, d).sum(1)
            x["k_cache"][b, :, n] = (qg * 100).to(x["k_cache"].dtype)
    out_dom = _run(x, scale).clone()
    assert torch.equal(out_nan.view(torch.int16), out_rand.view(torch.int16))
    assert torch.equal(out_nan.view(torch.int16), out_dom.view(torch.int16))
    for b, n in enumerate(lens):
        qg = x["q"][b].float().view(G, H // G, d).sum(1)
        x["k_cache"][b, :, n - 1] = (qg * 100).to(x["k_cache"].dtype)
        x["v_cache"][b, :, n - 1] = 2.0
    out_last = _run(x, scale)
    assert torch.equal(out_last, torch.full_like(out_last, 2.0))
    del x
    torch.cuda.empty_cache()


def _random_shapes(n, seed):
    """A fixed list of shapes drawn once from a seeded generator: every
    supported head size, group sizes from MQA to MHA, lengths from 0 to past
    the capacity, all three dtypes."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        n_rep = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 32]))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 5))
        n_max = int(rng.integers(1, 700))
        dt = str(rng.choice(["bf16", "f16", "f32"]))
        lens = [int(rng.integers(-2, n_max + 3)) for _ in range(B)]
        shapes.append((B, G * n_rep, G, d, n_max, dt, lens))
    return shapes


@pytest.mark.parametrize("case", _random_shapes(24, 2024))
def test_decode_random_shapes(case):
    B, H, G, d, n_max, dt, lens = case
    announce(f"decode random B={B} H={H} G={G} d={d} Nmax={n_max} {dt} lens={lens}")
    x = synth.decode_inputs(B, H, G, d, n_max, dtype=dt, seed=B + H + n_max, device=DEV,
                            seqlens=lens, nan_tail=False)
    scale = synth.scale_for(d)
    out = _run(x, scale)
    assert_close(out, _oracle(x, scale), x["q"].dtype, f"random {case}")


# float32 at scale 2: softmax arguments near 100 turn one float32 rounding of
# a score into a ~1e-5 relative change of its weight, so the fixed float32
# bound (set for scale 1/sqrt(d)) cannot hold there; that case is held to
# float32's own forward-error bound instead (f32_attention_bound)
@pytest.mark.parametrize("scale,dt", [(0.0, "bf16"), (-0.3, "bf16"), (2.0, "bf16"),
                                      (0.0, "f32"), (-0.3, "f32"), (2.0, "f32")])
def test_decode_unusual_scales(scale, dt):
    """scale 0 gives the plain mean of the attended V rows; a negative scale
    favours the least similar keys; a large one makes the softmax nearly hard
    (scores spread over dozens of powers of two)."""
    announce(f"decode scale={scale} {dt}")
    x = synth.decode_inputs(2, 32, 8, 128, 600, dtype=dt, seed=17, device=DEV, seqlens=[600, 345])
    got = _run(x, scale)
    ref = _oracle(x, scale)
    if dt == "f32" and scale == 2.0:
        q, k, v = to64(x["q"]), to64(x["k_cache"]), to64(x["v_cache"])
        n_rep = q.shape[1] // k.shape[1]
        g64 = to64(got)
        worst = 0.0
        for b, n in enumerate(x["seqlens"].cpu().tolist()):
            for h in range(q.shape[1]):
                g = h // n_rep
                exact, tol = f32_attention_bound(q[b, h][None], k[b, g, :n], v[b, g, :n], scale,
                                                 np.ones((1, n), dtype=bool))
                np.testing.assert_allclose(exact[0], ref[b, h], rtol=1e-12, atol=1e-13)
                err = np.abs(g64[b, h] - ref[b, h])
                assert (err <= tol[0]).all(), (b, h, float((err / tol[0]).max()))
                worst = max(worst, float((err / tol[0]).max()))
        print(f"decode f32 scale 2: largest error / bound = {worst:.3g}")
        return
    assert_close(got, ref, x["q"].dtype, f"scale={scale}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_split_merge_ignores_stale_workspace(dt):
    """The merge reads the partial slots of splits that did not run in this call
    (ragged lengths leave late splits empty); those slots hold whatever an
    earlier call left there.  Filled with NaN bit patterns (the arrival counters
    zeroed, as the library requires), the output must still be exact-to-tolerance
    and finite."""
    announce(f"decode stale workspace {dt}")
    B, H, G, d, n_max = 3, 32, 8, 128, 777
    x = synth.decode_inputs(B, H, G, d, n_max, dtype=dt, seed=23, device=DEV, seqlens=[777, 300, 5],
                            nan_tail=True)
    scale = synth.scale_for(d)
    need = gqa.decode_workspace_bytes(B, H, G, d, n_max, 0)
    assert need > 65536
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)     # float32 NaN everywhere
    ws[:65536] = 0                                                     # counter header
    out = gqa.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale, workspace=ws)
    torch.cuda.synchronize()
    assert_close(out, _oracle(x, scale), x["q"].dtype, "stale workspace")


def test_decode_on_two_streams():
    """Split decodes issued alternately on two streams (default priority) may run
    at the same time; each stream gets its own cached workspace, so both results
    are right."""
    announce("decode two streams")
    xa = synth.decode_inputs(4, 32, 8, 128, 900, dtype="bf16", seed=31, device=DEV, seqlens=[900, 513, 260, 7])
    xb = synth.decode_inputs(4, 32, 8, 128, 900, dtype="bf16", seed=32, device=DEV, seqlens=[31, 899, 700, 450])
    scale = synth.scale_for(128)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a, outs_b = [], []
    torch.cuda.synchronize()
    for _ in range(6):
        with torch.cuda.stream(sa):
            outs_a.append(gqa.decode(xa["q"], xa["k_cache"], xa["v_cache"], xa["seqlens"], scale=scale))
        with torch.cuda.stream(sb):
            outs_b.append(gqa.decode(xb["q"], xb["k_cache"], xb["v_cache"], xb["seqlens"], scale=scale))
    torch.cuda.synchronize()
    ra, rb = _oracle(xa, scale), _oracle(xb, scale)
    for oa, ob in zip(outs_a, outs_b):
        assert_close(oa, ra, torch.bfloat16, "stream a")
        assert_close(ob, rb, torch.bfloat16, "stream b")


def test_split_decode_beyond_counter_capacity():
    """More (sequence, K/V head) units than the workspace has arrival counters
    (16384): the split partials are then merged by the separate combine pass.
    Checked on sampled sequences."""
    announce("decode split, units beyond counter capacity")
    B, H, G, d, n_max = 2100, 32, 8, 64, 64
    rng = np.random.default_rng(5)
    lens = [int(v) for v in rng.integers(0, n_max + 1, B)]
    x = synth.decode_inputs(B, H, G, d, n_max, dtype="bf16", seed=41, device=DEV, seqlens=lens)
    scale = synth.scale_for(d)
    out = _run(x, scale, num_splits=2)
    rows = [0, 1, 2, 777, 1500, 2099] + [int(i) for i in rng.integers(0, B, 10)]
    assert_close(out[rows], _oracle(x, scale, rows=rows), torch.bfloat16, "combine pass")
