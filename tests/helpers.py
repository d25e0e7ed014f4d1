"""Shared helpers for the GPU parity tests (comparison against the float64 oracle)."""

import sys

import numpy as np
import pytest
import torch

# Tolerances for GPU vs float64 oracle on the same (rounded) inputs.
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 1.5e-2
BF16_MEAN_ABS = 2e-3
# IEEE half keeps 3 more mantissa bits than bfloat16 (the attention weights
# and the output are rounded to it): the bfloat16 bounds divided by 4.
F16_MAX_ABS = 4e-3
F16_MEAN_ABS = 5e-4


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def announce(msg: str) -> None:
    """Name the case on stdout before a GPU step (so a crash still says what ran)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def assert_close(got: torch.Tensor, ref: np.ndarray, dtype: torch.dtype, what: str = "") -> dict:
    g = to64(got)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if not np.isfinite(g).all():
        bad = np.argwhere(~np.isfinite(g))
        rows = sorted({tuple(int(i) for i in ix[:-1]) for ix in bad})
        raise AssertionError(f"{what}: non-finite output at {len(bad)} elements, "
                             f"rows (all indices but the last) {rows[:12]}{' ...' if len(rows) > 12 else ''}")
    err = np.abs(g - ref)
    stats = {"max_abs": float(err.max(initial=0.0)), "mean_abs": float(err.mean()) if err.size else 0.0}
    if dtype == torch.float32:
        assert stats["max_abs"] <= F32_MAX_ABS, f"{what}: {stats}"
    elif dtype == torch.float16:
        assert stats["max_abs"] <= F16_MAX_ABS and stats["mean_abs"] <= F16_MEAN_ABS, f"{what}: {stats}"
    else:
        assert stats["max_abs"] <= BF16_MAX_ABS and stats["mean_abs"] <= BF16_MEAN_ABS, f"{what}: {stats}"
    return stats


def bf16_ulp_distance(got_bf16: torch.Tensor, ref: np.ndarray) -> np.ndarray:
    """|bits(got) - bits(RNE_bf16(ref))| as integers (same-sign values assumed near)."""
    want = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
    a = got_bf16.detach().cpu().view(torch.int16).numpy().astype(np.int64)
    b = want.view(torch.int16).numpy().astype(np.int64)
    # map sign-magnitude to a monotone integer line
    a = np.where(a < 0, -(a & 0x7FFF), a)
    b = np.where(b < 0, -(b & 0x7FFF), b)
    return np.abs(a - b)


def f16_ulp_distance(got_f16: torch.Tensor, ref: np.ndarray) -> np.ndarray:
    """|bits(got) - bits(RNE_f16(ref))| as integers (same-sign values assumed near)."""
    want = torch.from_numpy(ref.astype(np.float32)).to(torch.float16)
    a = got_f16.detach().cpu().view(torch.int16).numpy().astype(np.int64)
    b = want.view(torch.int16).numpy().astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFF), a)
    b = np.where(b < 0, -(b & 0x7FFF), b)
    return np.abs(a - b)


def f32_attention_bound(q, K, V, scale, visible):
    """First-order forward-error bound of float32 softmax attention, per output
    element, evaluated with the exact (float64) weights.

    q [R, d]; K, V [n, d]; visible [R, n] (which positions each row attends).
    A float32 score carries at most gamma_d * |scale| * sum_c |q_c k_c| from
    its dot product (any summation order), plus a few roundings of the scale,
    the max subtraction and exp2; a relative error of at most delta on every
    weight moves the output by at most 2 delta sum_j p_j |v_j - out|, and the
    float32 weighted sum and its rescalings add gamma_n (sum_j p_j |v_j| + |out|).
    Returns (exact output, tolerance), both [R, d]."""
    u = 2.0 ** -24
    R, d = q.shape
    n_vis = visible.sum(axis=1)
    s = scale * (q @ K.T)
    sabs = abs(scale) * (np.abs(q) @ np.abs(K).T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.where(visible, np.exp(s - m), 0.0)
    p /= p.sum(axis=1, keepdims=True)
    out = p @ V
    gd = d * u / (1 - d * u)
    delta = (gd + 3 * u) * sabs + 2 * u * 1.4426950408889634 * np.abs(np.where(visible, s - m, 0.0)) + 4 * u
    dmax = np.where(visible, delta, 0.0).max(axis=1)
    spread = np.einsum("rj,rjc->rc", p, np.abs(V[None, :, :] - out[:, None, :]))
    gn = n_vis * u / (1 - n_vis * u)
    tol = 2 * dmax[:, None] * spread + gn[:, None] * (p @ np.abs(V) + np.abs(out)) + 2 * u * np.abs(out)
    return out, 1.1 * tol + 1e-12
