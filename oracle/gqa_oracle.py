"""Plain float64 CPU oracle for grouped-query attention (GQA).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg; never by the library.  It shares no code with
the HIP path and imports nothing from it.

Everything here is written to be checked by eye against the source pages, in
float64, one query head at a time, with explicit loops.  NumPy's ``@`` (a
matrix product) and ``np.exp`` serve as library steps; nothing is blocked,
fused or reordered beyond the definitions below.

Sources (cited by title and section):

* "GQA: Training Generalized Multi-Query Transformer Models from Multi-Head
  Checkpoints" (the GQA paper; Chinese translation on dtcms.com), sections
  2.1 (Uptraining, Figure 1) and 2.2 (Grouped-query attention, Figure 2).
* The 2kiu.com tutorial on MHA / MQA / GQA, sections 2.1, 3.1, 3.2, 4.1 and
  4.3 (the worked example of 8 heads in 2 groups, and the MHA-to-GQA
  conversion).
* The fogdragon CSDN blog post on MQA/GQA and the memory wall, sections
  "KV Cache" (the cached decode step written as two einsums around a softmax)
  and "MQA 的推导" (the per-step memory/arithmetic accounting for MHA and MQA).
* The CSDN interview explainer on GQA, section 03 (repeating each K/V head
  n_rep times so that an MHA kernel can be reused).

Readings taken where the pages are silent:

* Group membership is contiguous: query head h belongs to K/V head
  floor(h * G / H).  The tutorial's example puts heads 1-4 in group 1 and
  heads 5-8 in group 2; repeating each K/V head n_rep times in place gives the
  same assignment.
* H must be a multiple of G (every example on the pages divides evenly).
* ``scale`` is an argument; the pages divide the logits by sqrt(d) with d the
  per-head size.  Here the logits are multiplied by ``scale``.
* The decode step's own key is already in the cache (the blog concatenates the
  new k, v onto the cache before the attention), so a sequence of length n
  attends positions 0 .. n-1.  n = 0 gives a zero output; n > Nmax is clamped.
* Causal prefill: query position i attends keys 0 .. i inclusive.
* Decode with append: the new token's k, v go to cache position seqlens[b]-1
  (the length already counts the new token, as above), then the step attends
  0 .. seqlens[b]-1.  A length of 0 has no position for the token and a length
  above Nmax points past the cache: in both cases nothing is written (the
  attention itself then follows the decode rules above).
* Chunked prefill against a cache: a chunk of Tc new positions follows ctx
  cached ones (its own k, v already in the cache at ctx .. ctx+Tc-1, as for
  decode); chunk row t sits at absolute position ctx + t and attends positions
  0 .. ctx + t inclusive -- the causal rule of the prompt phase with an offset
  (Tc = 1 is the decode step, ctx = 0 the whole-prompt prefill).  Positions
  beyond the cache capacity Nmax are not attended (clamped); ctx < 0 reads as 0.
* GQKVA (the GQKVA summary on hub.baai.ac.cn): g_q query projections and g_kv
  key/value projections, attention for every (query group i, K/V group j)
  pair, g_q * g_kv outputs.  The pages do not fix the order of the outputs;
  here output head h pairs query group h // g_kv with K/V group h % g_kv
  (query-group-major).
* Mean-pooling is the arithmetic mean of the group's member heads.

Pins: every function here is checked against something other than itself
(library routines for the MHA/MQA/GQA special cases, closed forms, the pages'
printed numbers, brute force on tiny inputs) in tests/test_oracle_pins.py.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_group_of_head",
    "group_map",
    "attended_length",
    "softmax_weights",
    "attend_one_query",
    "decode_ref",
    "append_position",
    "decode_append_ref",
    "future_keys",
    "prefill_causal_ref",
    "chunk_attended_length",
    "prefill_chunk_ref",
    "gqkva_head_pair",
    "gqkva_decode_ref",
    "gqkva_prefill_causal_ref",
    "meanpool_ref",
    "kv_cache_values_per_token",
    "kv_cache_bytes",
    "kv_cache_reduction_factor",
    "decode_flops",
    "prefill_causal_flops",
]


# ---------------------------------------------------------------------------
# Head -> K/V-head grouping
# ---------------------------------------------------------------------------

def kv_group_of_head(h: int, H: int, G: int) -> int:
    """K/V head used by query head ``h`` (0-based) when H query heads share G K/V heads.

    GQA paper section 2.2: the query heads are divided into G groups and each
    group shares a single key head and a single value head; G = 1 is MQA and
    G = H is MHA.  Tutorial section 3.1 fixes the order with its example of 8
    heads in 2 groups (heads 1-4 use K_group1/V_group1, heads 5-8 use
    K_group2/V_group2), i.e. consecutive blocks of H/G heads.
    """
    if G < 1 or H < 1 or H % G != 0:
        raise ValueError(f"H={H} must be a positive multiple of G={G}")
    if not 0 <= h < H:
        raise ValueError(f"head {h} out of range for H={H}")
    n_rep = H // G
    return h // n_rep


def group_map(H: int, G: int) -> list[int]:
    """``[kv_group_of_head(h, H, G) for h in range(H)]``."""
    return [kv_group_of_head(h, H, G) for h in range(H)]


# ---------------------------------------------------------------------------
# Attention of one query over a cached K/V
# ---------------------------------------------------------------------------

def attended_length(seqlen: int, n_max: int) -> int:
    """Number of cached positions a decode query attends.

    The blog's "KV Cache" section appends the current token's k and v to the
    cache before the two einsums, so a sequence whose cache holds ``seqlen``
    entries (the current one included) attends all of them.  Lengths are
    clamped to [0, n_max].
    """
    return int(min(max(int(seqlen), 0), int(n_max)))


def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, in float64.

    The blog's "KV Cache" section normalises the logits with a softmax over
    the cached positions.  The maximum is subtracted first; in exact
    arithmetic that leaves the result unchanged, and it keeps exp() finite.
    Entries equal to -inf receive weight 0.
    """
    s = np.asarray(scores, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend_one_query(qvec: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K @ q) @ V for one query head.

    qvec: [d]; K, V: [n, d] (the positions this query attends, n >= 1).
    Blog "KV Cache" section: logits are the dot products of the query with
    every cached key, they are scaled and passed through a softmax over the
    positions, and the output is the weighted sum of the cached values.
    """
    qvec = np.asarray(qvec, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    logits = K @ qvec
    weights = softmax_weights(float(scale) * logits)
    return weights @ V


def decode_ref(q, k_cache, v_cache, seqlens, scale: float) -> np.ndarray:
    """One GQA decode step for a batch, in float64.  Returns out[B, H, d].

    q: [B, H, d]; k_cache, v_cache: [B, G, Nmax, d]; seqlens: [B] ints.
    For every sequence b and query head h, the head attends the first
    ``attended_length(seqlens[b], Nmax)`` cached positions of K/V head
    ``kv_group_of_head(h, H, G)`` (GQA paper section 2.2; blog "KV Cache"
    section for the attention itself).  A sequence with nothing cached gets a
    zero output.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    seqlens = np.asarray(seqlens).reshape(-1)
    B, H, d = q.shape
    Bk, G, n_max, dk = k_cache.shape
    if (Bk, dk) != (B, d) or v_cache.shape != k_cache.shape or seqlens.shape[0] != B:
        raise ValueError("inconsistent decode shapes")
    out = np.zeros((B, H, d), dtype=np.float64)
    for b in range(B):
        n = attended_length(seqlens[b], n_max)
        for h in range(H):
            g = kv_group_of_head(h, H, G)
            if n == 0:
                continue
            out[b, h] = attend_one_query(q[b, h], k_cache[b, g, :n], v_cache[b, g, :n], scale)
    return out


def append_position(seqlen: int, n_max: int):
    """Cache position that receives the new token's k and v, or None.

    The blog's "KV Cache" section concatenates the current step's k and v onto
    the cached K and V before the attention; with a cache of Nmax slots and a
    length that counts the new token, that is slot ``seqlen - 1``.  A length
    of 0 (no token) or above Nmax (no such slot) writes nothing.
    """
    seqlen = int(seqlen)
    if seqlen < 1 or seqlen > n_max:
        return None
    return seqlen - 1


def decode_append_ref(q, k_new, v_new, k_cache, v_cache, seqlens, scale: float):
    """Append the new token's k, v to the cache, then one decode step (float64).

    q: [B, H, d]; k_new, v_new: [B, G, d]; k_cache, v_cache: [B, G, Nmax, d].
    Returns (out [B, H, d], k_cache after, v_cache after); the inputs are not
    modified.  Blog "KV Cache" section: K = cat(K_prev, k), V = cat(V_prev, v),
    then softmax(q.K / sqrt(d)) V over the grown cache.
    """
    k_after = np.array(k_cache, dtype=np.float64, copy=True)
    v_after = np.array(v_cache, dtype=np.float64, copy=True)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    seqlens = np.asarray(seqlens).reshape(-1)
    B, G, n_max, d = k_after.shape
    if k_new.shape != (B, G, d) or v_new.shape != (B, G, d) or seqlens.shape[0] != B:
        raise ValueError("inconsistent append shapes")
    for b in range(B):
        pos = append_position(seqlens[b], n_max)
        if pos is None:
            continue
        for g in range(G):
            k_after[b, g, pos] = k_new[b, g]
            v_after[b, g, pos] = v_new[b, g]
    out = decode_ref(q, k_after, v_after, seqlens, scale)
    return out, k_after, v_after


def future_keys(rows, T: int) -> np.ndarray:
    """Boolean [len(rows), T]: True where key position j comes after query position i.

    Causal reading: position i sees keys 0..i (its own key included), so only
    j > i is hidden.
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    return np.arange(T)[None, :] > rows[:, None]


def prefill_causal_ref(q, k, v, scale: float, rows=None) -> np.ndarray:
    """Causal GQA over a whole prompt, in float64.  Returns out[B, T, H, d].

    q: [B, T, H, d]; k, v: [B, T, G, d] (token-major).  Query position i of
    head h attends keys 0..i (inclusive) of K/V head ``kv_group_of_head``.
    The blog describes the context phase as computed in parallel over the
    prompt, like an encoder, with each position seeing only its past; the
    attention per row is the same as in ``attend_one_query``.

    ``rows`` (optional) restricts the computation to those query positions;
    the other output rows are left as NaN.  The scores of a row are computed
    as one matrix product over all T keys; the keys after the row are then
    given weight 0 (their score is set to -inf before the softmax).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, d = q.shape
    G = k.shape[2]
    if k.shape != (B, T, G, d) or v.shape != k.shape:
        raise ValueError("inconsistent prefill shapes")
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    out = np.full((B, T, H, d), np.nan, dtype=np.float64)
    future = future_keys(rows, T)                             # [R, T]
    for b in range(B):
        for h in range(H):
            g = kv_group_of_head(h, H, G)
            Kbg = k[b, :, g, :]          # [T, d]
            Vbg = v[b, :, g, :]          # [T, d]
            logits = q[b, rows, h, :] @ Kbg.T            # [R, T]
            scores = float(scale) * logits
            scores = np.where(future, -np.inf, scores)
            out[b, rows, h, :] = softmax_weights(scores) @ Vbg
    return out


def chunk_attended_length(ctx: int, t: int, n_max: int) -> int:
    """Positions attended by row t of a chunk that follows ``ctx`` cached positions.

    The prompt phase's causal rule (a position sees itself and everything
    before it) with the chunk offset: absolute position ctx + t attends
    ctx + t + 1 positions, at most the ``n_max`` that exist.
    """
    ctx = max(int(ctx), 0)
    return int(min(ctx + int(t) + 1, int(n_max)))


def prefill_chunk_ref(q, k_cache, v_cache, ctx_lens, scale: float, rows=None) -> np.ndarray:
    """A prompt chunk attending the cache it extends, in float64.  Returns out[B, Tc, H, d].

    q: [B, Tc, H, d]; k_cache, v_cache: [B, G, Nmax, d] holding the ctx_lens[b]
    earlier positions and the chunk's own positions after them; ctx_lens: [B].
    Row t of sequence b, head h, attends the first
    ``chunk_attended_length(ctx_lens[b], t, Nmax)`` positions of K/V head
    ``kv_group_of_head(h, H, G)`` with ``attend_one_query``.  ``rows``
    (optional) restricts the computation to those chunk rows; the other output
    rows are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    ctx_lens = np.asarray(ctx_lens).reshape(-1)
    B, Tc, H, d = q.shape
    Bk, G, n_max, dk = k_cache.shape
    if (Bk, dk) != (B, d) or v_cache.shape != k_cache.shape or ctx_lens.shape[0] != B:
        raise ValueError("inconsistent chunk shapes")
    rows = range(Tc) if rows is None else [int(r) for r in np.asarray(rows).reshape(-1)]
    out = np.full((B, Tc, H, d), np.nan, dtype=np.float64)
    for b in range(B):
        for t in rows:
            n = chunk_attended_length(ctx_lens[b], t, n_max)
            for h in range(H):
                g = kv_group_of_head(h, H, G)
                if n == 0:
                    out[b, t, h] = 0.0
                    continue
                out[b, t, h] = attend_one_query(q[b, t, h], k_cache[b, g, :n], v_cache[b, g, :n], scale)
    return out


def gqkva_head_pair(h: int, g_q: int, g_kv: int) -> tuple[int, int]:
    """(query group, K/V group) of output head h under GQKVA (query-group-major)."""
    if g_q < 1 or g_kv < 1 or not 0 <= h < g_q * g_kv:
        raise ValueError("bad GQKVA head")
    return h // g_kv, h % g_kv


def gqkva_decode_ref(q, k_cache, v_cache, seqlens, scale: float) -> np.ndarray:
    """One GQKVA decode step, in float64.  Returns out[B, g_q * g_kv, d].

    q: [B, g_q, d] (one query per query group); k_cache, v_cache:
    [B, g_kv, Nmax, d].  Output head h = (i, j) = ``gqkva_head_pair`` attends
    the first ``attended_length`` cached positions of K/V group j with query
    group i's query (GQKVA summary: attention over every (Q, KV) combination).
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    seqlens = np.asarray(seqlens).reshape(-1)
    B, g_q, d = q.shape
    Bk, g_kv, n_max, dk = k_cache.shape
    if (Bk, dk) != (B, d) or v_cache.shape != k_cache.shape or seqlens.shape[0] != B:
        raise ValueError("inconsistent GQKVA decode shapes")
    out = np.zeros((B, g_q * g_kv, d), dtype=np.float64)
    for b in range(B):
        n = attended_length(seqlens[b], n_max)
        if n == 0:
            continue
        for h in range(g_q * g_kv):
            i, j = gqkva_head_pair(h, g_q, g_kv)
            out[b, h] = attend_one_query(q[b, i], k_cache[b, j, :n], v_cache[b, j, :n], scale)
    return out


def gqkva_prefill_causal_ref(q, k, v, scale: float, rows=None) -> np.ndarray:
    """Causal GQKVA over a prompt, in float64.  Returns out[B, T, g_q * g_kv, d].

    q: [B, T, g_q, d]; k, v: [B, T, g_kv, d].  Position t of output head
    h = (i, j) attends keys 0..t of K/V group j with query group i's query.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, g_q, d = q.shape
    g_kv = k.shape[2]
    if k.shape != (B, T, g_kv, d) or v.shape != k.shape:
        raise ValueError("inconsistent GQKVA prefill shapes")
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    out = np.full((B, T, g_q * g_kv, d), np.nan, dtype=np.float64)
    future = future_keys(rows, T)
    for b in range(B):
        for h in range(g_q * g_kv):
            i, j = gqkva_head_pair(h, g_q, g_kv)
            scores = float(scale) * (q[b, rows, i, :] @ k[b, :, j, :].T)
            scores = np.where(future, -np.inf, scores)
            out[b, rows, h, :] = softmax_weights(scores) @ v[b, :, j, :]
    return out


# ---------------------------------------------------------------------------
# MHA -> GQA checkpoint conversion
# ---------------------------------------------------------------------------

def meanpool_ref(w, G: int) -> np.ndarray:
    """Mean of each group's member heads, in float64.  w: [H, ...] -> [G, ...].

    GQA paper section 2.1 (Figure 1) and section 2.2: when a multi-head
    checkpoint is converted, each group's key (and value) projection matrix is
    the mean-pool of the projection matrices of all original heads in that
    group.  Tutorial section 4.3, step 2, says the same: average the key
    weight matrices of the heads in a group, and do the same for the value
    weights.  Groups are contiguous blocks of heads (``kv_group_of_head``).
    """
    w = np.asarray(w, dtype=np.float64)
    H = w.shape[0]
    if G < 1 or H % G != 0:
        raise ValueError(f"H={H} must be a positive multiple of G={G}")
    out = np.zeros((G,) + w.shape[1:], dtype=np.float64)
    counts = [0] * G
    for h in range(H):
        g = kv_group_of_head(h, H, G)
        out[g] += w[h]
        counts[g] += 1
    for g in range(G):
        out[g] /= counts[g]
    return out


# ---------------------------------------------------------------------------
# Accounting (sizes and operation counts), used by the pins and the tests
# ---------------------------------------------------------------------------

def kv_cache_values_per_token(n_kv_heads: int, head_dim: int, n_layers: int) -> int:
    """Cached values per token: a K and a V vector of every K/V head, in every layer.

    The blog's "KV Cache" section counts hidden size x 2 (K and V) x layers
    for an MHA model, whose K/V heads together span the hidden size.
    """
    return int(n_kv_heads) * int(head_dim) * 2 * int(n_layers)


def kv_cache_bytes(B: int, G: int, N: int, d: int, itemsize: int) -> int:
    """Bytes of one layer's K and V caches for B sequences of N positions."""
    return 2 * int(B) * int(G) * int(N) * int(d) * int(itemsize)


def kv_cache_reduction_factor(H: int, G: int) -> float:
    """How many times smaller the GQA-G cache is than the MHA (G = H) cache.

    GQA paper section 2.2: going from MHA to MQA reduces the K/V cache by a
    factor H; the tutorial gives 8x for 8-head MQA (section 2.1) and 4x for 8
    heads in 2 groups (section 3.1).
    """
    if G < 1 or H % G != 0:
        raise ValueError(f"H={H} must be a positive multiple of G={G}")
    return kv_cache_bytes(1, H, 1, 1, 1) / kv_cache_bytes(1, G, 1, 1, 1)


def decode_flops(H: int, total_positions: int, d: int) -> int:
    """Floating-point operations of one decode step (a multiply-add counts 2).

    The blog's "MQA 的推导" section counts b*h*n*d multiply-adds for the
    logits and the same again for the weighted sum of values, for MHA and for
    MQA alike: sharing K/V changes the bytes loaded, not the arithmetic.
    ``total_positions`` is the sum over sequences of the attended positions
    (b*n for a uniform batch).
    """
    return 4 * int(H) * int(total_positions) * int(d)


def prefill_causal_flops(B: int, T: int, H: int, d: int) -> int:
    """Operations of causal prefill counting only the attended (i, j <= i) pairs."""
    pairs = T * (T + 1) // 2
    return 2 * 2 * int(d) * int(B) * int(H) * int(pairs)
