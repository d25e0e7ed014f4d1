"""Seeded synthetic inputs for grouped-query attention workloads.

This module only draws random numbers and lays them out: it holds none of the
attention arithmetic, so both the HIP path's callers and the float64 oracle's
callers can take their inputs from here.  Every tensor is drawn with
``torch.Generator(device).manual_seed(seed)``; draws are made in a fixed order
(q, then K, then V, then the sequence lengths) so that the query is identical
across a sweep of the K/V-head count G.  Floating tensors are drawn in float32
from N(0, 1), multiplied by ``std`` when one is given, and then cast to the
requested dtype (bfloat16 casts round to nearest even).

The named workloads mirror the shapes of the pages' settings: a Llama-7B-sized
decoder layer (32 heads of 128), a T5-XXL-sized GQA-8 cross-attention step (64
heads of 64, encoder length 2048), long ragged caches, a 4096-token prompt.
The pages evaluate on summarisation, translation and QA datasets; those are
not used.  Random inputs of the same shapes stand in for them.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "scale_for",
    "decode_inputs",
    "decode_append_inputs",
    "prefill_inputs",
    "meanpool_inputs",
    "to_f64",
    "torch_dtype",
]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def scale_for(d: int) -> float:
    """The float32 number nearest 1/sqrt(d), as a Python float (the value every caller passes)."""
    return float(np.float32(1.0 / math.sqrt(d)))


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                      # "decode", "prefill" or "meanpool"
    dtype: str                     # "f32" or "bf16"
    B: int = 1
    H: int = 1
    G: int = 1
    d: int = 64
    N: int = 0                     # decode: Nmax; prefill: T
    seqlens: str = "full"          # decode: "full" (all = N) or "uniform" (U[1, N])
    nan_tail: bool = False         # decode: fill positions >= seqlen with NaN
    std: float = 1.0
    G_sweep: tuple = ()
    per_head_shape: tuple = ()     # meanpool: shape of one head's weights
    seed: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS: dict[str, Workload] = {
    "tiny_decode_f32": Workload(
        "tiny_decode_f32", "decode", "f32", B=1, H=8, G=2, d=64, N=128,
        G_sweep=(2, 8, 1),
        note="8 query heads in 2 groups (plus G=8 MHA and G=1 MQA), cache length 128"),
    "llama7b_decode_bf16": Workload(
        "llama7b_decode_bf16", "decode", "bf16", B=16, H=32, G=8, d=128, N=1024,
        G_sweep=(32, 8, 4, 1),
        note="Llama-7B-sized decode layer: 32 heads of 128, cache length 1024, batch 16"),
    "t5xxl_cross_decode_bf16": Workload(
        "t5xxl_cross_decode_bf16", "decode", "bf16", B=32, H=64, G=8, d=64, N=2048,
        note="T5-XXL-sized GQA-8 cross-attention step: 64 heads of 64, encoder length 2048"),
    "t5xxl_meanpool_bf16": Workload(
        "t5xxl_meanpool_bf16", "meanpool", "bf16", H=64, G=8, per_head_shape=(4096, 64),
        note="K/V projection weights [64 heads, 4096, 64] mean-pooled into 8 groups"),
    "ragged_longctx_decode_bf16": Workload(
        "ragged_longctx_decode_bf16", "decode", "bf16", B=64, H=32, G=8, d=128, N=32768,
        seqlens="uniform", nan_tail=True,
        note="ragged caches, lengths uniform in [1, 32768], NaN beyond each length"),
    "causal_prefill_bf16": Workload(
        "causal_prefill_bf16", "prefill", "bf16", B=2, H=32, G=8, d=128, N=4096, std=0.5,
        note="causal prefill of a 4096-token prompt, 32 heads of 128 in 8 groups"),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device, std, dtype):
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def decode_inputs(B, H, G, d, n_max, dtype="bf16", seed=0, device="cpu", seqlens="full",
                  nan_tail=False, std=1.0):
    """q[B,H,d], k_cache/v_cache[B,G,Nmax,d], seqlens[B] (int32).

    ``seqlens`` may be "full" (every sequence holds Nmax positions), "uniform"
    (lengths drawn uniformly from [1, Nmax], after V) or an explicit sequence
    of ints.  With ``nan_tail`` the cache positions at or beyond each length
    are set to NaN in K and V.
    """
    dt = torch_dtype(dtype) if isinstance(dtype, str) else dtype
    gen = _gen(device, seed)
    q = _randn((B, H, d), gen, device, std, dt)
    k = _randn((B, G, n_max, d), gen, device, std, dt)
    v = _randn((B, G, n_max, d), gen, device, std, dt)
    if isinstance(seqlens, str):
        if seqlens == "full":
            sl = torch.full((B,), n_max, dtype=torch.int32, device=device)
        elif seqlens == "uniform":
            sl = torch.randint(1, n_max + 1, (B,), generator=gen, device=device,
                               dtype=torch.int64).to(torch.int32)
        else:
            raise ValueError(seqlens)
    else:
        sl = torch.as_tensor(list(seqlens), dtype=torch.int32, device=device)
    if nan_tail:
        pos = torch.arange(n_max, device=device)
        tail = pos[None, :] >= sl.to(torch.int64)[:, None]          # [B, Nmax]
        tail = tail[:, None, :, None]
        k.masked_fill_(tail, float("nan"))
        v.masked_fill_(tail, float("nan"))
    return {"q": q, "k_cache": k, "v_cache": v, "seqlens": sl}


def decode_append_inputs(B, H, G, d, n_max, dtype="bf16", seed=0, device="cpu", seqlens="full",
                         nan_tail=False, std=1.0):
    """decode_inputs(...) plus this step's k_new, v_new [B,G,d], drawn after them
    from a generator of seed + 1_000_003 (so q and the caches match decode_inputs
    of the same seed)."""
    x = decode_inputs(B, H, G, d, n_max, dtype=dtype, seed=seed, device=device, seqlens=seqlens,
                      nan_tail=nan_tail, std=std)
    dt = x["q"].dtype
    gen = _gen(device, seed + 1_000_003)
    x["k_new"] = _randn((B, G, d), gen, device, std, dt)
    x["v_new"] = _randn((B, G, d), gen, device, std, dt)
    return x


def prefill_inputs(B, T, H, G, d, dtype="bf16", seed=0, device="cpu", std=0.5):
    """q[B,T,H,d], k/v[B,T,G,d] (token-major), drawn q then K then V."""
    dt = torch_dtype(dtype) if isinstance(dtype, str) else dtype
    gen = _gen(device, seed)
    q = _randn((B, T, H, d), gen, device, std, dt)
    k = _randn((B, T, G, d), gen, device, std, dt)
    v = _randn((B, T, G, d), gen, device, std, dt)
    return {"q": q, "k": k, "v": v}


def meanpool_inputs(H, per_head_shape, dtype="bf16", seed=0, device="cpu", std=1.0):
    """Per-head projection weights w[H, *per_head_shape]."""
    dt = torch_dtype(dtype) if isinstance(dtype, str) else dtype
    gen = _gen(device, seed)
    return {"w": _randn((H,) + tuple(per_head_shape), gen, device, std, dt)}


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy on the host of what a device tensor holds."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
