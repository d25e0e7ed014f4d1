"""GPU parity of gqa_decode_append (KV append fused into the decode step) against
the float64 oracle, through the C ABI binding."""

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


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns (NaN-safe exact comparison)."""
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def _run(x, scale, num_splits=0):
    k, v = x["k_cache"].clone(), x["v_cache"].clone()
    out = gqa.decode_append(x["q"], x["k_new"], x["v_new"], k, v, x["seqlens"], scale=scale,
                            num_splits=num_splits)
    torch.cuda.synchronize()
    return out, k, v


def _check_caches(x, k_after, v_after):
    """Row seqlens[b]-1 holds the new row bit for bit; every other element is unchanged."""
    n_max = x["k_cache"].shape[2]
    want_k, want_v = _bits(x["k_cache"]).copy(), _bits(x["v_cache"]).copy()
    kn, vn = _bits(x["k_new"]), _bits(x["v_new"])
    for b, n in enumerate(x["seqlens"].cpu().tolist()):
        pos = oracle.append_position(n, n_max)
        if pos is not None:
            want_k[b, :, pos] = kn[b]
            want_v[b, :, pos] = vn[b]
    assert np.array_equal(_bits(k_after), want_k)
    assert np.array_equal(_bits(v_after), want_v)


def _oracle(x, scale):
    out, _, _ = oracle.decode_append_ref(to64(x["q"]), to64(x["k_new"]), to64(x["v_new"]),
                                         to64(x["k_cache"]), to64(x["v_cache"]),
                                         x["seqlens"].cpu().numpy(), scale)
    return out


CASES = [
    # B, H, G, d, Nmax, dtype, lengths
    (4, 8, 2, 64, 300, "bf16", [1, 300, 257, 33]),
    (3, 32, 8, 128, 777, "bf16", [777, 513, 256]),
    (2, 32, 32, 128, 129, "bf16", [129, 65]),
    (2, 32, 1, 128, 600, "bf16", [600, 257]),
    (3, 64, 1, 64, 300, "bf16", [300, 1, 129]),          # four work groups share each K/V head
    (3, 64, 8, 64, 450, "bf16", [450, 1, 449]),
    (4, 24, 8, 128, 300, "bf16", [0, 301, 300, 2]),      # 0 and > Nmax write nothing
    (3, 8, 2, 64, 200, "f32", [200, 1, 77]),
    (2, 32, 8, 128, 130, "f32", [0, 131]),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}/{c[2]}x{c[3]}-N{c[4]}-{c[5]}" for c in CASES])
@pytest.mark.parametrize("num_splits", [0, 1, 3, 7])
def test_append_parity_and_cache(case, num_splits):
    B, H, G, d, n_max, dt, lens = case
    announce(f"decode_append {case} splits={num_splits}")
    x = synth.decode_append_inputs(B, H, G, d, n_max, dtype=dt, seed=B * 131 + H, device=DEV,
                                   seqlens=lens, nan_tail=True)
    scale = synth.scale_for(d)
    out, k_after, v_after = _run(x, scale, num_splits)
    _check_caches(x, k_after, v_after)
    assert_close(out, _oracle(x, scale), torch.float32 if dt == "f32" else torch.bfloat16,
                 f"append {case} S={num_splits}")


def test_append_split_boundaries_bf16():
    """Lengths whose new slot opens a split (the owning split has no cached row)."""
    B, H, G, d, n_max = 6, 32, 8, 128, 1024
    S = 4
    split_len = 256
    lens = [split_len + 1, 2 * split_len + 1, 3 * split_len + 1, split_len, 1, n_max]
    announce("decode_append split boundaries")
    x = synth.decode_append_inputs(B, H, G, d, n_max, seed=5, device=DEV, seqlens=lens, nan_tail=True)
    scale = synth.scale_for(d)
    out, k_after, v_after = _run(x, scale, num_splits=S)
    _check_caches(x, k_after, v_after)
    assert_close(out, _oracle(x, scale), torch.bfloat16, "split boundaries")


def test_append_single_token_is_exact():
    """Length 1: out is the group's new v exactly, whatever the cache holds."""
    B, H, G, d, n_max = 3, 32, 8, 128, 64
    announce("decode_append single token")
    x = synth.decode_append_inputs(B, H, G, d, n_max, seed=6, device=DEV, seqlens=[1, 1, 1],
                                   nan_tail=True)
    out, _, _ = _run(x, synth.scale_for(d))
    want = x["v_new"].repeat_interleave(H // G, dim=1)
    assert torch.equal(out, want)


def test_append_matches_write_then_decode():
    """Same function as writing the row and calling gqa.decode: bit-exact on the
    float32 path (same kernels), to tolerance on the fused bf16 path."""
    for dt in ("f32", "bf16"):
        B, H, G, d, n_max = 3, 16, 4, 128, 500
        announce(f"decode_append vs write+decode {dt}")
        x = synth.decode_append_inputs(B, H, G, d, n_max, dtype=dt, seed=7, device=DEV,
                                       seqlens=[500, 123, 1], nan_tail=True)
        scale = synth.scale_for(d)
        out, k_after, v_after = _run(x, scale)
        k2, v2 = x["k_cache"].clone(), x["v_cache"].clone()
        for b, n in enumerate(x["seqlens"].cpu().tolist()):
            k2[b, :, n - 1] = x["k_new"][b]
            v2[b, :, n - 1] = x["v_new"][b]
        ref = gqa.decode(x["q"], k2, v2, x["seqlens"], scale=scale)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(k_after), _bits(k2)) and np.array_equal(_bits(v_after), _bits(v2))
        if dt == "f32":
            assert torch.equal(out, ref)
        else:
            assert (out.float() - ref.float()).abs().max().item() <= 1.6e-2


def test_append_three_steps_chain():
    """Three decode steps in a row, each appending its token (lengths grow by one)."""
    B, H, G, d, n_max = 4, 32, 8, 128, 320
    announce("decode_append three-step chain")
    x = synth.decode_append_inputs(B, H, G, d, n_max, seed=8, device=DEV,
                                   seqlens=[255, 256, 1, 317], nan_tail=True)
    scale = synth.scale_for(d)
    k, v = x["k_cache"].clone(), x["v_cache"].clone()
    kr, vr = to64(k), to64(v)
    sl = x["seqlens"].clone()
    for step in range(3):
        y = synth.decode_append_inputs(B, H, G, d, 1, seed=100 + step, device=DEV)
        out = gqa.decode_append(y["q"], y["k_new"], y["v_new"], k, v, sl, scale=scale)
        torch.cuda.synchronize()
        ref, kr, vr = oracle.decode_append_ref(to64(y["q"]), to64(y["k_new"]), to64(y["v_new"]),
                                               kr, vr, sl.cpu().numpy(), scale)
        assert_close(out, ref, torch.bfloat16, f"chain step {step}")
        sl = sl + 1
    assert np.array_equal(to64(k)[~np.isnan(kr)], kr[~np.isnan(kr)])


def test_append_llama7b_full():
    w = synth.WORKLOADS["llama7b_decode_bf16"]
    announce("decode_append llama7b full size")
    x = synth.decode_append_inputs(w.B, w.H, w.G, w.d, w.N, seed=9, device=DEV, seqlens="uniform")
    scale = synth.scale_for(w.d)
    out, k_after, v_after = _run(x, scale)
    _check_caches(x, k_after, v_after)
    assert_close(out, _oracle(x, scale), torch.bfloat16, "llama7b append")
