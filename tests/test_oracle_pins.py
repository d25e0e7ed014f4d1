"""Pins for the float64 oracle: each check compares it with something other than itself.

* Library routines for the special cases the GQA paper (section 2.2) names:
  PyTorch's scaled_dot_product_attention in float64 on the CPU, for MHA
  (G = H), MQA (G = 1) and GQA (``enable_gqa=True``, which repeats each K/V
  head in place), and with ``is_causal`` for prefill.
* The pages' printed facts: the 8-heads-in-2-groups assignment and the K/V
  cache sizes (tests/golden/).
* Closed forms: one cached key, constant values, a zero query, two keys.
* Brute force with Python floats and math.exp on tiny inputs.
* Invariants: repeating K/V heads (the CSDN interview explainer, section 03),
  permuting cached positions, content beyond the sequence length.

The mutation tests at the end plant a plausible mistake in the oracle and check
that at least one pin catches it.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import gqa_oracle as og

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa_decode(q, k, v, seqlens, scale):
    """Reference decode through torch SDPA (float64, CPU), one sequence at a time."""
    B, H, d = q.shape
    out = np.zeros((B, H, d))
    for b in range(B):
        n = min(max(int(seqlens[b]), 0), k.shape[2])
        if n == 0:
            continue
        qb = torch.from_numpy(q[b][:, None, :].copy())              # [H, 1, d]
        kb = torch.from_numpy(k[b][:, :n, :].copy())                # [G, n, d]
        vb = torch.from_numpy(v[b][:, :n, :].copy())
        o = F.scaled_dot_product_attention(qb[None], kb[None], vb[None], scale=scale,
                                           enable_gqa=True)
        out[b] = o[0, :, 0, :].numpy()
    return out


# ---------------------------------------------------------------------------
# Pins written as plain functions, so that the mutation tests can call them too
# ---------------------------------------------------------------------------

def pin_golden_group_maps():
    with open(os.path.join(GOLDEN, "group_maps.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = [g + 1 for g in oracle.group_map(c["H"], c["G"])]
        assert got == c["group_of_head"], (c, got)


def pin_golden_kv_sizes():
    with open(os.path.join(GOLDEN, "kv_cache_sizes.json")) as f:
        gold = json.load(f)
    for r in gold["reduction"]:
        assert oracle.kv_cache_reduction_factor(r["H"], r["G"]) == r["factor"]
    L = gold["llama7b"]
    vals = oracle.kv_cache_values_per_token(L["n_heads"], L["head_dim"], L["n_layers"])
    assert L["n_heads"] * L["head_dim"] == L["hidden"]
    assert vals == L["values_per_token"]
    per_layer = oracle.kv_cache_bytes(1, L["n_heads"], 1, L["head_dim"], 2)
    assert per_layer * L["n_layers"] == L["bytes_per_token_half"]
    total = oracle.kv_cache_bytes(1, L["n_heads"], L["tokens"], L["head_dim"], 2) * L["n_layers"]
    assert total == L["bytes_total_half"]


def pin_decode_vs_sdpa(B=3, H=8, d=16, n_max=11, seed=0):
    rng = _rng(seed)
    scale = 0.37
    for G in [g for g in range(1, H + 1) if H % g == 0]:
        q = rng.standard_normal((B, H, d))
        k = rng.standard_normal((B, G, n_max, d))
        v = rng.standard_normal((B, G, n_max, d))
        seqlens = [n_max, 1, 7][:B]
        ref = _sdpa_decode(q, k, v, seqlens, scale)
        got = oracle.decode_ref(q, k, v, seqlens, scale)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def pin_mha_vs_sdpa_no_grouping(B=2, H=4, d=8, n=9, seed=1):
    """G = H against SDPA called as plain multi-head attention (no GQA flag)."""
    rng = _rng(seed)
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[:, :, None], torch.from_numpy(k),
                                         torch.from_numpy(v), scale=0.5)[:, :, 0].numpy()
    got = oracle.decode_ref(q, k, v, [n] * B, 0.5)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def pin_mqa_vs_sdpa_broadcast(B=2, H=6, d=8, n=9, seed=2):
    """G = 1 against SDPA with the single K/V head broadcast over all heads."""
    rng = _rng(seed)
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, 1, n, d))
    v = rng.standard_normal((B, 1, n, d))
    kt = torch.from_numpy(k).expand(B, H, n, d)
    vt = torch.from_numpy(v).expand(B, H, n, d)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[:, :, None], kt, vt,
                                         scale=0.25)[:, :, 0].numpy()
    got = oracle.decode_ref(q, k, v, [n] * B, 0.25)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def _brute_decode(q, k, v, seqlens, scale):
    B, H, d = len(q), len(q[0]), len(q[0][0])
    G, n_max = len(k[0]), len(k[0][0])
    out = [[[0.0] * d for _ in range(H)] for _ in range(B)]
    for b in range(B):
        n = min(max(int(seqlens[b]), 0), n_max)
        for h in range(H):
            g = h * G // H
            if n == 0:
                continue
            s = []
            for j in range(n):
                acc = 0.0
                for c in range(d):
                    acc += q[b][h][c] * k[b][g][j][c]
                s.append(scale * acc)
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for c in range(d):
                out[b][h][c] = sum(e[j] * v[b][g][j][c] for j in range(n)) / z
    return out


def pin_brute_force(seed=3):
    rng = _rng(seed)
    for H in (1, 2, 4):
        for G in [g for g in (1, 2, 4) if g <= H and H % g == 0]:
            for d in (1, 3, 4):
                B, n_max = 2, 5
                q = rng.standard_normal((B, H, d))
                k = rng.standard_normal((B, G, n_max, d))
                v = rng.standard_normal((B, G, n_max, d))
                seqlens = rng.integers(0, n_max + 2, size=B)
                ref = np.array(_brute_decode(q.tolist(), k.tolist(), v.tolist(), seqlens, 0.7))
                got = oracle.decode_ref(q, k, v, seqlens, 0.7)
                np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def pin_single_key(seed=4):
    rng = _rng(seed)
    B, H, G, d, n_max = 3, 8, 2, 16, 6
    q = rng.standard_normal((B, H, d)) * 10
    k = rng.standard_normal((B, G, n_max, d))
    v = rng.standard_normal((B, G, n_max, d))
    got = oracle.decode_ref(q, k, v, [1] * B, 0.3)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(got[b, h], v[b, h // (H // G), 0])


def pin_constant_values(seed=5):
    rng = _rng(seed)
    B, H, G, d, n_max = 2, 8, 4, 8, 17
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, G, n_max, d))
    c = rng.standard_normal((B, G, 1, d))
    v = np.broadcast_to(c, (B, G, n_max, d)).copy()
    got = oracle.decode_ref(q, k, v, [n_max, 9], 0.5)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(got[b, h], c[b, h // (H // G), 0], rtol=1e-14, atol=0)


def pin_zero_query_is_mean(seed=6):
    rng = _rng(seed)
    B, H, G, d, n = 2, 4, 2, 8, 16
    q = np.zeros((B, H, d))
    k = rng.standard_normal((B, G, n, d))
    v = rng.standard_normal((B, G, n, d))
    got = oracle.decode_ref(q, k, v, [n, 8], 1.0)
    for b, nb in enumerate([n, 8]):
        for h in range(H):
            np.testing.assert_allclose(got[b, h], v[b, h // 2, :nb].mean(axis=0), rtol=1e-14,
                                       atol=1e-15)


def pin_two_keys_sigmoid(seed=7):
    rng = _rng(seed)
    d = 4
    for _ in range(20):
        q = rng.standard_normal((1, 1, d))
        k = rng.standard_normal((1, 1, 2, d))
        v = rng.standard_normal((1, 1, 2, d))
        scale = 0.9
        delta = scale * (q[0, 0] @ k[0, 0, 1] - q[0, 0] @ k[0, 0, 0])
        w1 = 1.0 / (1.0 + math.exp(-delta))
        expect = w1 * v[0, 0, 1] + (1.0 - w1) * v[0, 0, 0]
        got = oracle.decode_ref(q, k, v, [2], scale)[0, 0]
        np.testing.assert_allclose(got, expect, rtol=1e-13, atol=1e-15)


def pin_repeat_kv(seed=8):
    """GQA-G equals MHA on K/V heads each repeated n_rep times in place."""
    rng = _rng(seed)
    B, H, d, n_max = 2, 8, 8, 13
    for G in (1, 2, 4):
        q = rng.standard_normal((B, H, d))
        k = rng.standard_normal((B, G, n_max, d))
        v = rng.standard_normal((B, G, n_max, d))
        seqlens = [13, 5]
        kr = np.repeat(k, H // G, axis=1)
        vr = np.repeat(v, H // G, axis=1)
        a = oracle.decode_ref(q, k, v, seqlens, 0.4)
        b = oracle.decode_ref(q, kr, vr, seqlens, 0.4)
        np.testing.assert_allclose(a, b, rtol=1e-15, atol=0)


def pin_tail_ignored(seed=9):
    rng = _rng(seed)
    B, H, G, d, n_max = 3, 4, 2, 8, 10
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, G, n_max, d))
    v = rng.standard_normal((B, G, n_max, d))
    seqlens = [3, 10, 1]
    base = oracle.decode_ref(q, k, v, seqlens, 0.5)
    k2, v2 = k.copy(), v.copy()
    for b, s in enumerate(seqlens):
        k2[b, :, s:] = np.nan
        v2[b, :, s:] = np.nan
    nanfill = oracle.decode_ref(q, k2, v2, seqlens, 0.5)
    assert np.array_equal(base, nanfill)
    # a dominant key just inside the length must win; one just outside must not
    k3 = k.copy()
    v3 = v.copy()
    b = 0
    s = seqlens[b]
    k3[b, :, s - 1] = 50.0 * q[b, 0] / np.linalg.norm(q[b, 0])
    v3[b, :, s - 1] = 7.0
    out3 = oracle.decode_ref(q, k3, v3, seqlens, 1.0)
    np.testing.assert_allclose(out3[b, 0], 7.0, rtol=0, atol=1e-12)


def pin_permutation(seed=10):
    rng = _rng(seed)
    B, H, G, d, n = 1, 4, 2, 8, 12
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, G, n, d))
    v = rng.standard_normal((B, G, n, d))
    perm = rng.permutation(n)
    a = oracle.decode_ref(q, k, v, [n], 0.5)
    b = oracle.decode_ref(q, k[:, :, perm], v[:, :, perm], [n], 0.5)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def pin_prefill_vs_sdpa(seed=11):
    rng = _rng(seed)
    B, T, H, d = 2, 9, 8, 8
    for G in (1, 2, 8):
        q = rng.standard_normal((B, T, H, d))
        k = rng.standard_normal((B, T, G, d))
        v = rng.standard_normal((B, T, G, d))
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q).transpose(1, 2), torch.from_numpy(k).transpose(1, 2),
            torch.from_numpy(v).transpose(1, 2), is_causal=True, scale=0.3,
            enable_gqa=True).transpose(1, 2).numpy()
        got = oracle.prefill_causal_ref(q, k, v, 0.3)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def pin_prefill_rows_are_decodes(seed=12):
    rng = _rng(seed)
    B, T, H, G, d = 2, 7, 4, 2, 8
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, G, d))
    v = rng.standard_normal((B, T, G, d))
    full = oracle.prefill_causal_ref(q, k, v, 0.6)
    kc = np.ascontiguousarray(k.transpose(0, 2, 1, 3))      # [B, G, T, d]
    vc = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    for i in range(T):
        dec = oracle.decode_ref(q[:, i], kc, vc, [i + 1] * B, 0.6)
        np.testing.assert_allclose(full[:, i], dec, rtol=1e-13, atol=1e-14)
    # row 0 attends only key 0
    for h in range(H):
        assert np.array_equal(full[:, 0, h], v[:, 0, h // (H // G)])
    rows = oracle.prefill_causal_ref(q, k, v, 0.6, rows=[0, 5])
    assert np.array_equal(rows[:, [0, 5]], full[:, [0, 5]])
    assert np.isnan(rows[:, 1]).all()


def pin_meanpool(seed=13):
    rng = _rng(seed)
    H, r, c = 8, 5, 3
    w = rng.standard_normal((H, r, c))
    assert np.array_equal(oracle.meanpool_ref(w, H), w)                 # G = H: identity
    np.testing.assert_allclose(oracle.meanpool_ref(w, 1)[0], w.mean(axis=0), rtol=1e-14,
                               atol=1e-15)                              # G = 1: global mean
    for G in (2, 4):
        ref = w.reshape(G, H // G, r, c).mean(axis=1)                    # library mean
        np.testing.assert_allclose(oracle.meanpool_ref(w, G), ref, rtol=1e-14, atol=1e-15)
    same = np.broadcast_to(w[:1], w.shape).copy() * 0.75                # identical heads
    assert np.array_equal(oracle.meanpool_ref(same, 2)[1], same[0])
    # the group of head h is floor(h*G/H): group 1 of 8-in-2 is heads 4..7
    marks = np.zeros((H, 1))
    marks[4:] = 1.0
    assert np.array_equal(oracle.meanpool_ref(marks, 2)[:, 0], [0.0, 1.0])


def pin_append_vs_sdpa_concat(seed=15):
    """Blog "KV Cache": K = cat(K_prev, k), V = cat(V_prev, v), then the attention
    over the grown cache -- built with torch.cat and run through SDPA (float64)."""
    rng = _rng(seed)
    B, H, G, d, n_max = 4, 8, 2, 16, 9
    scale = 1.0 / math.sqrt(d)
    q = rng.standard_normal((B, H, d))
    kc = rng.standard_normal((B, G, n_max, d))
    vc = rng.standard_normal((B, G, n_max, d))
    k_new = rng.standard_normal((B, G, d))
    v_new = rng.standard_normal((B, G, d))
    seqlens = [1, 5, 9, 3]
    out, _, _ = oracle.decode_append_ref(q, k_new, v_new, kc, vc, seqlens, scale)
    for b in range(B):
        n = seqlens[b]
        K = torch.cat([torch.from_numpy(kc[b, :, :n - 1]), torch.from_numpy(k_new[b])[:, None]], dim=1)
        V = torch.cat([torch.from_numpy(vc[b, :, :n - 1]), torch.from_numpy(v_new[b])[:, None]], dim=1)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[b])[None, :, None], K[None], V[None],
                                             scale=scale, enable_gqa=True)[0, :, 0]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)


def pin_append_cache_rows(seed=16):
    """The new k, v land in slot seqlens[b]-1; no other slot changes (NaN stays NaN);
    a length of 0 or above Nmax writes nothing."""
    rng = _rng(seed)
    B, H, G, d, n_max = 5, 4, 2, 8, 6
    kc = rng.standard_normal((B, G, n_max, d))
    kc[:, :, 4:] = np.nan
    vc = kc * 2.0
    k_new = rng.standard_normal((B, G, d))
    v_new = rng.standard_normal((B, G, d))
    seqlens = [3, 1, 6, 0, 7]
    q = rng.standard_normal((B, H, d))
    _, ka, va = oracle.decode_append_ref(q, k_new, v_new, kc, vc, seqlens, 0.5)
    for b, n in enumerate(seqlens):
        for g in range(G):
            for j in range(n_max):
                if 1 <= n <= n_max and j == n - 1:
                    assert np.array_equal(ka[b, g, j], k_new[b, g]) and np.array_equal(va[b, g, j], v_new[b, g])
                else:
                    assert np.array_equal(ka[b, g, j], kc[b, g, j], equal_nan=True)
                    assert np.array_equal(va[b, g, j], vc[b, g, j], equal_nan=True)


def pin_append_single_token(seed=17):
    """Length 1: the only attended key is the new one, so every head returns its
    group's new v exactly (whatever the cache holds)."""
    rng = _rng(seed)
    B, H, G, d, n_max = 2, 6, 3, 5, 4
    q = rng.standard_normal((B, H, d))
    kc = np.full((B, G, n_max, d), np.nan)
    k_new = rng.standard_normal((B, G, d))
    v_new = rng.standard_normal((B, G, d))
    out, _, _ = oracle.decode_append_ref(q, k_new, v_new, kc, kc, [1, 1], 0.3)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(out[b, h], v_new[b, h // (H // G)])


def pin_chunk_vs_sdpa_mask(seed=18):
    """A chunk after ctx cached positions: SDPA with an explicit boolean mask in
    which row t may see positions 0 .. ctx+t (float64, CPU)."""
    rng = _rng(seed)
    B, H, G, d, n_max, Tc = 4, 8, 2, 16, 20, 5
    scale = 1.0 / math.sqrt(d)
    q = rng.standard_normal((B, Tc, H, d))
    kc = rng.standard_normal((B, G, n_max, d))
    vc = rng.standard_normal((B, G, n_max, d))
    ctx = [0, 7, 15, 18]                    # the last one runs past the cache: clamped
    out = oracle.prefill_chunk_ref(q, kc, vc, ctx, scale)
    for b in range(B):
        L = min(ctx[b] + Tc, n_max)
        mask = torch.zeros((Tc, L), dtype=torch.bool)
        for t in range(Tc):
            mask[t, :min(ctx[b] + t, n_max - 1) + 1] = True
        qb = torch.from_numpy(q[b].transpose(1, 0, 2).copy())[None]          # [1, H, Tc, d]
        kb = torch.from_numpy(kc[b, :, :L].copy())[None]                     # [1, G, L, d]
        vb = torch.from_numpy(vc[b, :, :L].copy())[None]
        ref = F.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(out[b], ref[0].numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def pin_chunk_single_row_is_decode(seed=19):
    """A one-position chunk is the decode step with length ctx + 1."""
    rng = _rng(seed)
    B, H, G, d, n_max = 3, 8, 4, 8, 12
    q = rng.standard_normal((B, 1, H, d))
    kc = rng.standard_normal((B, G, n_max, d))
    vc = rng.standard_normal((B, G, n_max, d))
    ctx = [0, 5, 11]
    out = oracle.prefill_chunk_ref(q, kc, vc, ctx, 0.4)
    ref = _sdpa_decode(q[:, 0], kc, vc, [c + 1 for c in ctx], 0.4)
    np.testing.assert_allclose(out[:, 0], ref, rtol=1e-12, atol=1e-12)


def pin_chunk_zero_ctx_is_prefill(seed=20):
    """ctx = 0 with the prompt's K/V in the cache is the whole-prompt causal prefill
    (torch SDPA with is_causal)."""
    rng = _rng(seed)
    B, T, H, G, d = 2, 9, 6, 3, 8
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, G, T, d))
    v = rng.standard_normal((B, G, T, d))
    out = oracle.prefill_chunk_ref(q, k, v, [0, 0], 0.3)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q.transpose(0, 2, 1, 3).copy()),
                                         torch.from_numpy(k), torch.from_numpy(v), is_causal=True,
                                         scale=0.3, enable_gqa=True)
    np.testing.assert_allclose(out, ref.numpy().transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-12)


def _expand_gqkva(q, k, g_q, g_kv, axis_q, axis_k):
    """MHA operands of GQKVA: head h takes query group h // g_kv and K/V group h % g_kv."""
    qi = [h // g_kv for h in range(g_q * g_kv)]
    kj = [h % g_kv for h in range(g_q * g_kv)]
    return np.take(q, qi, axis=axis_q), np.take(k, kj, axis=axis_k)


def pin_gqkva_vs_sdpa_expanded(seed=21):
    """GQKVA decode and prefill against plain MHA (torch SDPA) on operands expanded
    to one (query, K/V) pair per output head."""
    rng = _rng(seed)
    B, g_q, g_kv, d, n_max = 3, 2, 3, 8, 10
    q = rng.standard_normal((B, g_q, d))
    kc = rng.standard_normal((B, g_kv, n_max, d))
    vc = rng.standard_normal((B, g_kv, n_max, d))
    sl = [10, 4, 1]
    out = oracle.gqkva_decode_ref(q, kc, vc, sl, 0.35)
    qe, ke = _expand_gqkva(q, kc, g_q, g_kv, 1, 1)
    _, ve = _expand_gqkva(q, vc, g_q, g_kv, 1, 1)
    np.testing.assert_allclose(out, _sdpa_decode(qe, ke, ve, sl, 0.35), rtol=1e-12, atol=1e-12)
    T = 7
    qp = rng.standard_normal((B, T, g_q, d))
    kp = rng.standard_normal((B, T, g_kv, d))
    vp = rng.standard_normal((B, T, g_kv, d))
    outp = oracle.gqkva_prefill_causal_ref(qp, kp, vp, 0.35)
    qe, ke = _expand_gqkva(qp, kp, g_q, g_kv, 2, 2)
    _, ve = _expand_gqkva(qp, vp, g_q, g_kv, 2, 2)
    ref = F.scaled_dot_product_attention(torch.from_numpy(qe.transpose(0, 2, 1, 3).copy()),
                                         torch.from_numpy(ke.transpose(0, 2, 1, 3).copy()),
                                         torch.from_numpy(ve.transpose(0, 2, 1, 3).copy()),
                                         is_causal=True, scale=0.35)
    np.testing.assert_allclose(outp, ref.numpy().transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-12)


def pin_gqkva_special_cases(seed=22):
    """Constant V per K/V group j: every head paired with j returns that constant.
    One query group (MKVA): heads differ only in their K/V group."""
    rng = _rng(seed)
    B, g_q, g_kv, d, n_max = 2, 3, 2, 4, 6
    q = rng.standard_normal((B, g_q, d))
    kc = rng.standard_normal((B, g_kv, n_max, d))
    vc = np.empty((B, g_kv, n_max, d))
    vc[:, 0] = 0.25
    vc[:, 1] = -1.5
    out = oracle.gqkva_decode_ref(q, kc, vc, [6, 3], 0.5)
    for h in range(g_q * g_kv):
        np.testing.assert_allclose(out[:, h], np.full((B, d), 0.25 if h % g_kv == 0 else -1.5),
                                   rtol=1e-14, atol=0)
    v2 = rng.standard_normal((B, g_kv, n_max, d))
    q1 = q[:, :1]
    out1 = oracle.gqkva_decode_ref(q1, kc, v2, [6, 3], 0.5)
    for j in range(g_kv):
        for b, n in enumerate([6, 3]):
            want = oracle.attend_one_query(q1[b, 0], kc[b, j, :n], v2[b, j, :n], 0.5)
            assert np.array_equal(out1[b, j], want)


def pin_flop_counts():
    # Decode operations do not depend on G (blog, "MQA 的推导": the arithmetic is unchanged)
    assert oracle.decode_flops(32, 16 * 1024, 128) == 268435456
    # Causal prefill: count attended pairs one by one on a small case
    B, T, H, d = 2, 13, 3, 8
    pairs = sum(1 for i in range(T) for j in range(T) if j <= i)
    assert oracle.prefill_causal_flops(B, T, H, d) == B * H * pairs * 2 * 2 * d


PINS = [
    pin_golden_group_maps, pin_golden_kv_sizes, pin_decode_vs_sdpa, pin_mha_vs_sdpa_no_grouping,
    pin_mqa_vs_sdpa_broadcast, pin_brute_force, pin_single_key, pin_constant_values,
    pin_zero_query_is_mean, pin_two_keys_sigmoid, pin_repeat_kv, pin_tail_ignored,
    pin_permutation, pin_prefill_vs_sdpa, pin_prefill_rows_are_decodes, pin_meanpool,
    pin_append_vs_sdpa_concat, pin_append_cache_rows, pin_append_single_token,
    pin_chunk_vs_sdpa_mask, pin_chunk_single_row_is_decode, pin_chunk_zero_ctx_is_prefill,
    pin_gqkva_vs_sdpa_expanded, pin_gqkva_special_cases, pin_flop_counts,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_group_map_rejects_indivisible():
    with pytest.raises(ValueError):
        oracle.kv_group_of_head(0, 6, 4)
    with pytest.raises(ValueError):
        oracle.meanpool_ref(np.zeros((6, 2)), 4)


def test_zero_length_gives_zero():
    q = np.ones((2, 2, 4))
    k = np.full((2, 1, 3, 4), np.nan)
    out = oracle.decode_ref(q, k, k, [0, 0], 1.0)
    assert np.array_equal(out, np.zeros_like(out))


def test_length_beyond_cache_is_clamped():
    rng = _rng(14)
    q = rng.standard_normal((1, 2, 4))
    k = rng.standard_normal((1, 1, 3, 4))
    v = rng.standard_normal((1, 1, 3, 4))
    assert np.array_equal(oracle.decode_ref(q, k, v, [99], 1.0), oracle.decode_ref(q, k, v, [3], 1.0))


# ---------------------------------------------------------------------------
# Mutation tests: plant a mistake in the oracle and make sure a pin fails
# ---------------------------------------------------------------------------

def _fails(pins):
    failed = []
    for p in pins:
        try:
            p()
        except (AssertionError, ValueError, IndexError):
            failed.append(p.__name__)
    return failed


def _mutant_attend(mutation):
    def attend(qvec, K, V, scale):
        qvec = np.asarray(qvec, dtype=np.float64)
        K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64)
        if mutation == "no_scale":
            s = K @ qvec
        elif mutation == "keys_as_values":
            s = scale * (K @ qvec)
            w = og.softmax_weights(s)
            return w @ K
        elif mutation == "divide_by_scale":
            s = (K @ qvec) / scale
        else:
            raise ValueError(mutation)
        return og.softmax_weights(s) @ V
    return attend


@pytest.mark.parametrize("mutation", ["no_scale", "keys_as_values", "divide_by_scale"])
def test_mutation_attention_caught(monkeypatch, mutation):
    monkeypatch.setattr(og, "attend_one_query", _mutant_attend(mutation))
    assert _fails([pin_decode_vs_sdpa, pin_brute_force, pin_two_keys_sigmoid])


def test_mutation_group_map_modulo_caught(monkeypatch):
    monkeypatch.setattr(og, "kv_group_of_head", lambda h, H, G: h % G)
    failed = _fails([pin_golden_group_maps, pin_decode_vs_sdpa, pin_repeat_kv, pin_meanpool])
    assert "pin_golden_group_maps" in failed and "pin_decode_vs_sdpa" in failed


def test_mutation_off_by_one_length_caught(monkeypatch):
    monkeypatch.setattr(og, "attended_length", lambda s, n: int(min(max(int(s) - 1, 0), n)))
    assert _fails([pin_single_key, pin_brute_force, pin_decode_vs_sdpa])


def test_mutation_softmax_without_normalisation_caught(monkeypatch):
    def bad(scores):
        s = np.asarray(scores, dtype=np.float64)
        return np.exp(s - np.max(s, axis=-1, keepdims=True))
    monkeypatch.setattr(og, "softmax_weights", bad)
    assert _fails([pin_constant_values, pin_decode_vs_sdpa, pin_prefill_vs_sdpa])


# (an exclusive mask leaves row 0 with no key: its softmax is NaN, as the pin expects)
@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
def test_mutation_causal_mask_exclusive_caught(monkeypatch):
    monkeypatch.setattr(og, "future_keys",
                        lambda rows, T: np.arange(T)[None, :] >= np.asarray(rows)[:, None])
    assert _fails([pin_prefill_vs_sdpa, pin_prefill_rows_are_decodes])


def test_mutation_causal_mask_missing_caught(monkeypatch):
    monkeypatch.setattr(og, "future_keys",
                        lambda rows, T: np.zeros((len(np.asarray(rows)), T), dtype=bool))
    assert _fails([pin_prefill_vs_sdpa, pin_prefill_rows_are_decodes])


def test_mutation_meanpool_sum_caught(monkeypatch):
    orig = og.meanpool_ref
    monkeypatch.setattr(oracle, "meanpool_ref", lambda w, G: orig(w, G) * (np.asarray(w).shape[0] // G))
    assert _fails([pin_meanpool]) == ["pin_meanpool"]


def test_mutation_append_off_by_one_caught(monkeypatch):
    monkeypatch.setattr(og, "append_position", lambda s, n: int(s) if 0 <= int(s) < n else None)
    failed = _fails([pin_append_vs_sdpa_concat, pin_append_cache_rows, pin_append_single_token])
    assert "pin_append_vs_sdpa_concat" in failed and "pin_append_cache_rows" in failed


def test_mutation_append_skipped_caught(monkeypatch):
    monkeypatch.setattr(og, "append_position", lambda s, n: None)
    failed = _fails([pin_append_vs_sdpa_concat, pin_append_cache_rows, pin_append_single_token])
    assert len(failed) == 3


def test_mutation_chunk_off_by_one_caught(monkeypatch):
    monkeypatch.setattr(og, "chunk_attended_length",
                        lambda c, t, n: int(min(max(int(c), 0) + int(t), int(n))))
    failed = _fails([pin_chunk_vs_sdpa_mask, pin_chunk_single_row_is_decode, pin_chunk_zero_ctx_is_prefill])
    assert len(failed) == 3


def test_mutation_gqkva_pairing_swapped_caught(monkeypatch):
    monkeypatch.setattr(og, "gqkva_head_pair", lambda h, gq, gkv: (h % gq, h // gq))
    failed = _fails([pin_gqkva_vs_sdpa_expanded, pin_gqkva_special_cases])
    assert "pin_gqkva_vs_sdpa_expanded" in failed and "pin_gqkva_special_cases" in failed
