"""GPU parity of chunked prefill against a cache (gqa_prefill_chunk) and of GQKVA
decode / prefill against the float64 oracle, through the C ABI binding."""

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


def _chunk_inputs(B, T, H, G, d, n_max, ctx, dt, seed):
    """Cache [B,G,Nmax,d] with NaN after each chunk's last position; queries [B,T,H,d]."""
    x = synth.decode_inputs(B, H, G, d, n_max, dtype=dt, seed=seed, device=DEV)
    ends = torch.tensor([min(max(c, 0) + T, n_max) for c in ctx], device=DEV)
    tail = (torch.arange(n_max, device=DEV)[None, :] >= ends[:, None])[:, None, :, None]
    x["k_cache"].masked_fill_(tail, float("nan"))
    x["v_cache"].masked_fill_(tail, float("nan"))
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed + 77)
    q = torch.randn((B, T, H, d), generator=gen, device=DEV, dtype=torch.float32).to(x["q"].dtype)
    return q, x["k_cache"], x["v_cache"], torch.tensor(ctx, dtype=torch.int32, device=DEV)


CHUNK_CASES = [
    # B, T, H, G, d, Nmax, ctx, dtype
    (3, 100, 8, 2, 128, 600, [0, 250, 500], "bf16"),
    (2, 257, 32, 8, 128, 1100, [31, 843], "bf16"),
    (2, 64, 8, 8, 64, 300, [100, 236], "bf16"),          # n_rep = 1
    (2, 70, 8, 4, 64, 400, [5, 300], "bf16"),            # n_rep = 2
    (1, 40, 32, 1, 128, 200, [150], "bf16"),             # n_rep = 32
    (2, 33, 24, 8, 128, 300, [7, 200], "bf16"),          # n_rep = 3: one padded head quad
    (2, 60, 12, 2, 128, 300, [40, 200], "bf16"),         # n_rep = 6: second quad half padded
    (3, 50, 8, 2, 128, 120, [100, -4, 70], "bf16"),      # past the cache (clamped), negative ctx
    (2, 1, 32, 8, 128, 500, [0, 499], "bf16"),           # one row: a decode step
    (2, 90, 8, 2, 128, 300, [10, 200], "f16"),
    (2, 70, 16, 4, 64, 400, [33, 250], "f16"),         # d = 64, n_rep = 4
    (2, 45, 8, 2, 64, 200, [20, 150], "f32"),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=[str(i) for i in range(len(CHUNK_CASES))])
def test_prefill_chunk_parity(case):
    B, T, H, G, d, n_max, ctx, dt = case
    announce(f"prefill_chunk {case}")
    q, kc, vc, cl = _chunk_inputs(B, T, H, G, d, n_max, ctx, dt, seed=T + n_max)
    scale = synth.scale_for(d)
    out = gqa.prefill_chunk(q, kc, vc, cl, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.prefill_chunk_ref(to64(q), to64(kc), to64(vc), ctx, scale)
    assert_close(out, ref, q.dtype, f"chunk {case}")


def test_prefill_chunk_zero_ctx_equals_prefill_bit_exact():
    """ctx = 0 with the prompt in the cache runs the same tiles as gqa_prefill_causal."""
    B, T, H, G, d = 2, 333, 32, 8, 128
    announce("prefill_chunk ctx=0 vs prefill_causal")
    x = synth.prefill_inputs(B, T, H, G, d, dtype="bf16", seed=5, device=DEV)
    ref = gqa.prefill_causal(x["q"], x["k"], x["v"], scale=0.09)
    kc = x["k"].transpose(1, 2).contiguous()
    vc = x["v"].transpose(1, 2).contiguous()
    out = gqa.prefill_chunk(x["q"], kc, vc, torch.zeros(B, dtype=torch.int32, device=DEV), scale=0.09)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_prefill_chunk_pieces_equal_whole_prompt():
    """A prompt prefilled in three chunks gives the whole-prompt result (to tolerance)."""
    B, T, H, G, d = 2, 600, 32, 8, 128
    announce("prefill_chunk three pieces")
    x = synth.prefill_inputs(B, T, H, G, d, dtype="bf16", seed=6, device=DEV)
    whole = gqa.prefill_causal(x["q"], x["k"], x["v"], scale=0.09)
    kc = x["k"].transpose(1, 2).contiguous()
    vc = x["v"].transpose(1, 2).contiguous()
    pieces = []
    for c0, c1 in ((0, 100), (100, 357), (357, 600)):
        cl = torch.full((B,), c0, dtype=torch.int32, device=DEV)
        pieces.append(gqa.prefill_chunk(x["q"][:, c0:c1].contiguous(), kc, vc, cl, scale=0.09))
    torch.cuda.synchronize()
    got = torch.cat(pieces, dim=1)
    assert (got.float() - whole.float()).abs().max().item() <= 1.6e-2


def test_prefill_chunk_full_size_sampled_rows():
    """4096-token context, a 2048-token chunk after a 2048-token prefix."""
    B, T, H, G, d, n_max = 2, 2048, 32, 8, 128, 4096
    announce("prefill_chunk full size")
    q, kc, vc, cl = _chunk_inputs(B, T, H, G, d, n_max, [2048, 1000], "bf16", seed=7)
    out = gqa.prefill_chunk(q, kc, vc, cl, scale=synth.scale_for(d))
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 1000, 2047]
    ref = oracle.prefill_chunk_ref(to64(q), to64(kc), to64(vc), [2048, 1000], synth.scale_for(d), rows=rows)
    assert_close(out[:, rows], ref[:, rows], torch.bfloat16, "chunk full size")


GQKVA_DECODE = [
    # B, g_q, g_kv, d, Nmax, lengths, splits, dtype
    (3, 2, 3, 128, 500, [500, 77, 1], 0, "bf16"),
    (2, 3, 2, 64, 300, [300, 150], 3, "bf16"),
    (2, 1, 6, 128, 200, [200, 5], 0, "bf16"),            # MKVA: one query group
    (2, 6, 1, 128, 250, [250, 0], 2, "bf16"),
    (2, 32, 4, 128, 400, [400, 399], 0, "bf16"),
    (2, 40, 2, 64, 100, [100, 60], 0, "bf16"),           # 40 queries per K/V head: vector units
    (2, 2, 3, 128, 300, [300, 120], 0, "f16"),
    (2, 3, 2, 64, 150, [150, 33], 4, "f32"),
]


@pytest.mark.parametrize("case", GQKVA_DECODE, ids=[str(i) for i in range(len(GQKVA_DECODE))])
def test_gqkva_decode_parity(case):
    B, g_q, g_kv, d, n_max, lens, S, dt = case
    announce(f"gqkva_decode {case}")
    # g_q query heads against g_kv K/V heads (any ratio), NaN beyond each length
    x = synth.decode_inputs(B, g_q, g_kv, d, n_max, dtype=dt, seed=g_q * 10 + g_kv, device=DEV,
                            seqlens=lens, nan_tail=True)
    scale = synth.scale_for(d)
    out = gqa.gqkva_decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale, num_splits=S)
    torch.cuda.synchronize()
    ref = oracle.gqkva_decode_ref(to64(x["q"]), to64(x["k_cache"]), to64(x["v_cache"]),
                                  x["seqlens"].cpu().numpy(), scale)
    assert_close(out, ref, x["q"].dtype, f"gqkva decode {case}")


def test_gqkva_decode_matches_expanded_mha():
    """GQKVA equals MHA (gqa.decode with G = H) on operands expanded to one
    (query, K/V) pair per output head."""
    B, g_q, g_kv, d, n_max = 2, 3, 4, 128, 300
    announce("gqkva_decode vs expanded MHA")
    x = synth.decode_inputs(B, 12, 4, d, n_max, seed=9, device=DEV, seqlens=[300, 123])
    q = x["q"][:, :g_q].contiguous()
    out = gqa.gqkva_decode(q, x["k_cache"], x["v_cache"], x["seqlens"], scale=0.1)
    heads = g_q * g_kv
    qi = torch.tensor([h // g_kv for h in range(heads)], device=DEV)
    kj = torch.tensor([h % g_kv for h in range(heads)], device=DEV)
    ref = gqa.decode(q[:, qi].contiguous(), x["k_cache"][:, kj].contiguous(),
                     x["v_cache"][:, kj].contiguous(), x["seqlens"], scale=0.1)
    torch.cuda.synchronize()
    assert (out.float() - ref.float()).abs().max().item() <= 1.6e-2


GQKVA_PREFILL = [
    # B, T, g_q, g_kv, d, dtype
    (2, 150, 2, 3, 128, "bf16"),
    (1, 200, 4, 2, 64, "bf16"),
    (2, 97, 1, 6, 128, "bf16"),
    (1, 130, 3, 2, 128, "bf16"),        # 3 queries per K/V head: one padded quad
    (1, 90, 5, 2, 64, "bf16"),          # 5 queries per K/V head: second quad padded
    (2, 100, 2, 3, 128, "f16"),
    (1, 70, 2, 3, 64, "f32"),
]


@pytest.mark.parametrize("case", GQKVA_PREFILL, ids=[str(i) for i in range(len(GQKVA_PREFILL))])
def test_gqkva_prefill_parity(case):
    B, T, g_q, g_kv, d, dt = case
    announce(f"gqkva_prefill {case}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(T + g_q)
    tdt = synth.torch_dtype(dt)
    q = (0.5 * torch.randn((B, T, g_q, d), generator=gen, device=DEV)).to(tdt)
    k = (0.5 * torch.randn((B, T, g_kv, d), generator=gen, device=DEV)).to(tdt)
    v = (0.5 * torch.randn((B, T, g_kv, d), generator=gen, device=DEV)).to(tdt)
    scale = synth.scale_for(d)
    out = gqa.gqkva_prefill_causal(q, k, v, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.gqkva_prefill_causal_ref(to64(q), to64(k), to64(v), scale)
    assert_close(out, ref, tdt, f"gqkva prefill {case}")
