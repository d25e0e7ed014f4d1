"""GPU parity of the IEEE-half (float16) paths -- decode, decode with append,
causal prefill, mean-pool -- against the float64 oracle on the same rounded
inputs, through the C ABI binding."""

import numpy as np
import pytest
import torch

import grouped_query_decode_amd as gqa
import oracle
import synth
from helpers import announce, assert_close, f16_ulp_distance, need_gpu, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F16 = torch.float16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    gqa.load_library()


DECODE_CASES = [
    # B, H, G, d, Nmax, lengths, splits
    (3, 8, 2, 64, 300, [300, 1, 77], 0),
    (2, 32, 8, 128, 777, [777, 300], 0),
    (2, 32, 8, 128, 777, [777, 300], 5),
    (2, 32, 32, 128, 129, [129, 2], 0),
    (2, 32, 1, 128, 600, [600, 0], 3),
    (2, 64, 8, 64, 450, [450, 449], 2),
    (2, 24, 8, 128, 200, [200, 150], 0),     # n_rep = 3
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(i) for i in range(len(DECODE_CASES))])
def test_decode_f16(case):
    B, H, G, d, n_max, lens, S = case
    announce(f"decode f16 {case}")
    x = synth.decode_inputs(B, H, G, d, n_max, dtype="f16", seed=B + H + n_max, device=DEV,
                            seqlens=lens, nan_tail=True)
    scale = synth.scale_for(d)
    out = gqa.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale, num_splits=S)
    torch.cuda.synchronize()
    assert out.dtype == F16
    ref = oracle.decode_ref(to64(x["q"]), to64(x["k_cache"]), to64(x["v_cache"]),
                            x["seqlens"].cpu().numpy(), scale)
    assert_close(out, ref, F16, f"decode f16 {case}")


def test_decode_f16_llama7b_full():
    w = synth.WORKLOADS["llama7b_decode_bf16"]
    announce("decode f16 llama7b full size")
    x = synth.decode_inputs(w.B, w.H, w.G, w.d, w.N, dtype="f16", seed=0, device=DEV)
    scale = synth.scale_for(w.d)
    out = gqa.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale)
    torch.cuda.synchronize()
    ref = oracle.decode_ref(to64(x["q"]), to64(x["k_cache"]), to64(x["v_cache"]),
                            x["seqlens"].cpu().numpy(), scale)
    assert_close(out, ref, F16, "decode f16 llama7b")


def test_decode_f16_single_key_and_constant_v_exact():
    announce("decode f16 exact cases")
    B, H, G, d, n_max = 2, 32, 8, 128, 256
    x = synth.decode_inputs(B, H, G, d, n_max, dtype="f16", seed=3, device=DEV, seqlens=[1, 256])
    v = x["v_cache"].clone()
    v[1] = 0.375
    out = gqa.decode(x["q"], x["k_cache"], v, x["seqlens"], scale=synth.scale_for(d))
    torch.cuda.synchronize()
    assert torch.equal(out[0], v[0, :, 0].repeat_interleave(H // G, dim=0))
    assert torch.equal(out[1], torch.full_like(out[1], 0.375))


def test_decode_append_f16():
    announce("decode_append f16")
    B, H, G, d, n_max = 4, 32, 8, 128, 500
    x = synth.decode_append_inputs(B, H, G, d, n_max, dtype="f16", seed=11, device=DEV,
                                   seqlens=[500, 257, 1, 0], nan_tail=True)
    scale = synth.scale_for(d)
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    out = gqa.decode_append(x["q"], x["k_new"], x["v_new"], kc, vc, x["seqlens"], scale=scale,
                            num_splits=2)
    torch.cuda.synchronize()
    ref, k_ref, v_ref = oracle.decode_append_ref(to64(x["q"]), to64(x["k_new"]), to64(x["v_new"]),
                                                 to64(x["k_cache"]), to64(x["v_cache"]),
                                                 x["seqlens"].cpu().numpy(), scale)
    assert_close(out, ref, F16, "decode_append f16")
    got_k = to64(kc)
    assert np.array_equal(got_k, k_ref, equal_nan=True)
    assert np.array_equal(to64(vc), v_ref, equal_nan=True)


PREFILL_CASES = [
    # B, T, H, G, d
    (2, 200, 8, 2, 128),
    (1, 333, 32, 8, 128),
    (2, 130, 8, 8, 64),
    (2, 97, 8, 4, 64),
    (1, 150, 32, 1, 128),
    (1, 64, 24, 8, 128),       # n_rep = 3: one padded head quad
]


@pytest.mark.parametrize("B,T,H,G,d", PREFILL_CASES)
def test_prefill_f16(B, T, H, G, d):
    announce(f"prefill f16 B={B} T={T} H={H} G={G} d={d}")
    x = synth.prefill_inputs(B, T, H, G, d, dtype="f16", seed=T + H + 1, device=DEV, std=0.5)
    scale = synth.scale_for(d)
    out = gqa.prefill_causal(x["q"], x["k"], x["v"], scale=scale)
    torch.cuda.synchronize()
    ref = oracle.prefill_causal_ref(to64(x["q"]), to64(x["k"]), to64(x["v"]), scale)
    assert_close(out, ref, F16, "prefill f16")
    assert torch.equal(out[:, 0], x["v"][:, 0].repeat_interleave(H // G, dim=1))


def test_prefill_f16_full_size_sampled_rows():
    w = synth.WORKLOADS["causal_prefill_bf16"]
    announce("prefill f16 full size")
    x = synth.prefill_inputs(w.B, w.N, w.H, w.G, w.d, dtype="f16", seed=1, device=DEV, std=w.std)
    scale = synth.scale_for(w.d)
    out = gqa.prefill_causal(x["q"], x["k"], x["v"], scale=scale)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 1000, 2047, 2048, 4095]
    ref = oracle.prefill_causal_ref(to64(x["q"]), to64(x["k"]), to64(x["v"]), scale, rows=rows)
    assert_close(out[:, rows], ref[:, rows], F16, "prefill f16 full size")


@pytest.mark.parametrize("H,G,shape", [(64, 8, (4096, 64)), (8, 2, (5, 3)), (6, 3, (7, 5))])
def test_meanpool_f16(H, G, shape):
    announce(f"meanpool f16 H={H} G={G} {shape}")
    w = synth.meanpool_inputs(H, shape, dtype="f16", seed=H * G, device=DEV)["w"]
    out = gqa.meanpool_heads(w, G)
    torch.cuda.synchronize()
    ulps = f16_ulp_distance(out, oracle.meanpool_ref(to64(w), G))
    assert ulps.max() <= 1, ulps.max()
