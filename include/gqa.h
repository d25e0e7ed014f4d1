/*
 * gqa.h - C ABI of libgqa.so: grouped-query attention on AMD MI355X (gfx950).
 *
 * Grouped-query attention (GQA paper, "GQA: Training Generalized Multi-Query
 * Transformer Models from Multi-Head Checkpoints", section 2.2): H query heads
 * are split into G groups and every group shares one key head and one value
 * head.  G = H is multi-head attention, G = 1 is multi-query attention.  Query
 * head h uses K/V head floor(h * G / H): the groups are consecutive blocks of
 * n_rep = H / G heads, as in the 2kiu.com MHA/MQA/GQA tutorial's example of 8
 * heads in 2 groups (section 3.1: heads 1-4 share group 1, heads 5-8 group 2).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensor arguments are DEVICE pointers owned by the caller, dense and
 *   row-major in the shapes given below, each 16-byte aligned.  The library
 *   never allocates, frees or keeps them after the call returns.
 * - dtype is GQA_DTYPE_F32 (float), GQA_DTYPE_BF16 (bfloat16) or GQA_DTYPE_F16
 *   (IEEE half); inputs and outputs share it.  Arithmetic is float32
 *   throughout; a 16-bit output is rounded once, to nearest even.  On the
 *   16-bit paths the attention weights are rounded to the same 16-bit format
 *   before they multiply V (the matrix cores take 16-bit operands).
 * - stream is a hipStream_t passed as void* (NULL: the null stream).  Work is
 *   enqueued asynchronously on it; the library never synchronises.  A fault
 *   inside a kernel surfaces at the caller's next synchronisation.
 * - Arguments are checked on the host before anything is enqueued: an invalid
 *   call returns a non-zero gqa_status, touches no memory and enqueues nothing;
 *   gqa_last_error() then gives a readable reason (per thread).
 * - Calls that only need host-side checks (an invalid argument, or an empty
 *   problem, which returns GQA_OK) make no HIP call at all.
 * - Every call is reentrant: no global state besides the per-thread error
 *   text.  Calls that share a workspace must not overlap in time.
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of every tensor argument of a call (inputs and outputs share
 * it).  Passed by value; an int-sized enum, so callers through a plain C FFI
 * may pass the int codes. */
typedef enum gqa_dtype {
  GQA_DTYPE_F32 = 0,         /* float                                          */
  GQA_DTYPE_BF16 = 1,        /* bfloat16 (top half of a float, round to even)  */
  GQA_DTYPE_F16 = 2          /* IEEE 754 binary16                              */
} gqa_dtype;

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1,   /* shapes, pointers, alignment, scale, H % G != 0   */
  GQA_ERR_UNSUPPORTED = 2,   /* valid, but not built: head size other than 64/128 */
  GQA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required        */
  GQA_ERR_LAUNCH = 4         /* the HIP runtime refused a kernel launch, or the
                                library's own objects disagree on the size of an
                                internal argument structure (a build from mixed
                                sources); nothing is enqueued in the latter case */
} gqa_status;

/*
 * Split planning for gqa_decode.
 *
 * A decode call divides each sequence's cache into num_splits slices, runs
 * one pass per slice and, when num_splits > 1, merges the slices' partial
 * softmax results (log-sum-exp): inside the same launch (the last slice of a
 * (sequence, K/V head) to finish merges), or in a second launch when there are
 * more than 16384 (sequence, K/V head) pairs or the float32 path runs.  The
 * partial results live in a caller-provided workspace.
 *
 * gqa_decode_num_splits() returns the split count gqa_decode() uses.  It is a
 * pure function of the shape (it reads no device and no sequence length), so
 * it and gqa_decode_workspace_bytes() can be called without a GPU.
 * Returns 0 for an invalid shape.
 *
 * gqa_decode_workspace_bytes(): bytes of workspace that a decode of this
 * shape needs with num_splits slices (num_splits = 0: the planner's choice).
 * 0 means no workspace is needed.  Returns (size_t)-1 for an invalid shape.
 *
 * Workspace contract: a device buffer, 16-byte aligned.  Its first 64 KiB hold
 * one arrival counter per (sequence, K/V head), which lets the last split to
 * finish merge the others inside the same kernel launch.  The caller
 * zero-fills the buffer ONCE before its first use (e.g. hipMemset at
 * allocation); every completed call leaves those 64 KiB zero again, so the
 * same buffer can then be reused for any shape without clearing.  Calls that
 * share a workspace must not overlap in time (use one workspace per stream).
 */
int gqa_decode_num_splits(int B, int H, int G, int d, int n_max);
size_t gqa_decode_workspace_bytes(int B, int H, int G, int d, int n_max, int num_splits);

/*
 * gqa_decode - one autoregressive decode step of GQA over a K/V cache.
 *
 * Defines (the fogdragon CSDN blog on MQA/GQA, section "KV Cache": the new
 * token's k and v are appended to the cache, then the query attends every
 * cached position through softmax(logits * scale) and a weighted sum of the
 * cached values; GQA paper section 2.2 for the head grouping):
 *
 *   out[b,h,:] = sum_{j < n_b} softmax_j(scale * q[b,h,:] . K[b,g,j,:]) V[b,g,j,:]
 *   with g = floor(h * G / H) and n_b = min(seqlens[b], n_max).
 *
 *   q        [B, H, d]          dtype, device
 *   k_cache  [B, G, n_max, d]   dtype, device
 *   v_cache  [B, G, n_max, d]   dtype, device
 *   seqlens  [B]                int32, device; the current token's K/V is
 *                               already at position seqlens[b]-1.  A length of
 *                               0 (or below) gives a zero output row; lengths
 *                               above n_max are clamped to n_max.  Cache rows
 *                               at or beyond the length are never read into
 *                               arithmetic (they may hold anything, NaN too).
 *   out      [B, H, d]          dtype, device; written in full.
 *   scale    finite float, typically 1/sqrt(d).
 *   d        64 or 128 (anything else: GQA_ERR_UNSUPPORTED).
 *   workspace/workspace_bytes   device buffer of at least
 *                               gqa_decode_workspace_bytes(B,H,G,d,n_max,0)
 *                               bytes, zero-filled before its first use (see
 *                               the workspace contract above); may be NULL/0
 *                               when that size is 0.
 *
 * Errors: GQA_ERR_INVALID_ARG for B, H, G, n_max < 0 or H, G < 1 with B > 0,
 * H % G != 0, a NULL or misaligned tensor, an unknown dtype or a non-finite
 * scale; GQA_ERR_WORKSPACE for a too-small workspace.  B = 0 or n_max = 0 with
 * B > 0 (then out is zero-filled) are valid.
 */
gqa_status gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seqlens, void* out,
                      int B, int H, int G, int d, int n_max, float scale, gqa_dtype dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_decode_split - gqa_decode with an explicit split count (1 .. n_max;
 * 0 = the planner's choice).  Needs gqa_decode_workspace_bytes(..., num_splits)
 * bytes of workspace.  Every split count computes the same function; only the
 * order of the floating-point sums changes.
 */
gqa_status gqa_decode_split(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seqlens, void* out,
                            int B, int H, int G, int d, int n_max, float scale, gqa_dtype dtype,
                            int num_splits, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * gqa_decode_append - append this step's k, v to the caches, then decode, in
 * one call (one kernel launch on the 16-bit paths).
 *
 * Defines (the fogdragon CSDN blog, section "KV Cache": each step
 * concatenates its new k and v onto the cached K and V -- K = cat(K_prev, k),
 * V = cat(V_prev, v) -- and then attends the grown cache):
 *
 *   if 1 <= seqlens[b] <= n_max:
 *       k_cache[b,g,seqlens[b]-1,:] = k_new[b,g,:];  v_cache[...] = v_new[b,g,:]
 *   then out = gqa_decode(q, k_cache, v_cache, seqlens)  (same definition).
 *
 *   k_new, v_new  [B, G, d]        dtype, device, read only.
 *   k_cache, v_cache [B, G, n_max, d]  dtype, device; exactly the row
 *                  seqlens[b]-1 of each (b, g) is written (a copy of the new
 *                  row, bit for bit); nothing is written for a length of 0
 *                  (no token) or above n_max (no such slot), and those
 *                  sequences decode as gqa_decode would.  Every other cache
 *                  element is left untouched.
 *   num_splits     as in gqa_decode_split (0 = the planner's choice).
 *   Other arguments, workspace contract and errors: as gqa_decode_split;
 *   k_new or v_new NULL (with B > 0) or misaligned is GQA_ERR_INVALID_ARG.
 *   The result equals writing the rows and then calling gqa_decode, up to the
 *   order of the floating-point sums.
 */
gqa_status gqa_decode_append(const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* seqlens, void* out,
                             int B, int H, int G, int d, int n_max, float scale, gqa_dtype dtype,
                             int num_splits, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * gqa_prefill_causal - causal GQA over whole prompts (the context phase).
 *
 * The blog's decoder discussion: the prompt is processed in parallel like an
 * encoder, but each position only sees itself and earlier positions.  Query
 * position i of head h attends keys 0..i (inclusive) of K/V head
 * floor(h * G / H):
 *
 *   out[b,i,h,:] = sum_{j <= i} softmax_j(scale * q[b,i,h,:] . k[b,j,g,:]) v[b,j,g,:]
 *
 *   q    [B, T, H, d]   dtype, device (token-major)
 *   k    [B, T, G, d]   dtype, device
 *   v    [B, T, G, d]   dtype, device
 *   out  [B, T, H, d]   dtype, device; written in full.
 *   d    64 or 128.
 *
 * bfloat16 and IEEE half run on the matrix cores (16-bit products, float32
 * accumulation; the softmax weights are rounded to the 16-bit format before
 * they multiply V, and the normaliser sums those rounded weights).  float32
 * runs on the vector units in float32.  Errors as for gqa_decode; B = 0 or T = 0 is a valid no-op.
 */
gqa_status gqa_prefill_causal(const void* q, const void* k, const void* v, void* out,
                              int B, int T, int H, int G, int d, float scale, gqa_dtype dtype,
                              void* stream);

/*
 * gqa_prefill_chunk - a chunk of a prompt attending the cache it extends
 * (chunked prefill).
 *
 * The prompt phase's causal rule -- each position sees itself and every
 * earlier position (the blog's decoder discussion; gqa_prefill_causal) -- for
 * T new positions that follow ctx_lens[b] positions already in the cache.  As
 * in gqa_decode, the chunk's own K/V are already written, at cache positions
 * ctx_lens[b] .. ctx_lens[b] + T - 1:
 *
 *   out[b,t,h,:] = sum_{j <= a} softmax_j(scale * q[b,t,h,:] . K[b,g,j,:]) V[b,g,j,:]
 *   with g = floor(h * G / H), a = min(ctx_lens[b] + t, n_max - 1).
 *
 *   q        [B, T, H, d]       dtype, device
 *   k_cache  [B, G, n_max, d]   dtype, device (the gqa_decode layout)
 *   v_cache  [B, G, n_max, d]
 *   ctx_lens [B] int32, device: cached positions before the chunk (negative
 *            reads as 0).  Rows whose position would pass the cache are
 *            clamped to the last slot.  Positions after a row's own are
 *            never read into its arithmetic.
 *   out      [B, T, H, d]       dtype, device; written in full.
 *   n_max >= 1.  T = 1 is a decode step with seqlens = ctx_lens + 1; ctx = 0
 *   with the prompt in the cache is gqa_prefill_causal.  Errors as for
 *   gqa_prefill_causal (ctx_lens NULL is GQA_ERR_INVALID_ARG).
 */
gqa_status gqa_prefill_chunk(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* ctx_lens, void* out,
                             int B, int T, int H, int G, int d, int n_max, float scale, gqa_dtype dtype,
                             void* stream);

/*
 * GQKVA - grouped queries AND grouped keys/values (the GQKVA summary on
 * hub.baai.ac.cn): g_q query projections and g_kv key/value projections, one
 * attention for every (query group i, K/V group j) pair, g_q * g_kv outputs.
 * Output head h pairs query group i = h / g_kv with K/V group j = h % g_kv
 * (query-group-major; the pages do not fix the order).  g_q = 1 is MKVA.
 *
 * gqkva_decode: q [B, g_q, d]; k_cache, v_cache [B, g_kv, n_max, d];
 *   seqlens as in gqa_decode; out [B, g_q * g_kv, d]:
 *   out[b,h,:] = sum_{j < n_b} softmax_j(scale * q[b,i,:] . K[b,j',j,:]) V[b,j',j,:]
 *   with (i, j') the pair of h.  Each K/V row is read once for all g_q
 *   queries.  Workspace: gqkva_decode_workspace_bytes() (same contract as
 *   gqa_decode's); num_splits as in gqa_decode_split.
 * gqkva_prefill_causal: q [B, T, g_q, d]; k, v [B, T, g_kv, d];
 *   out [B, T, g_q * g_kv, d]; position t attends keys 0..t.
 * Errors as for gqa_decode / gqa_prefill_causal (g_q, g_kv >= 1; any ratio).
 */
gqa_status gqkva_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens, void* out,
                        int B, int g_q, int g_kv, int d, int n_max, float scale, gqa_dtype dtype,
                        int num_splits, void* workspace, size_t workspace_bytes, void* stream);
size_t gqkva_decode_workspace_bytes(int B, int g_q, int g_kv, int d, int n_max, int num_splits);
gqa_status gqkva_prefill_causal(const void* q, const void* k, const void* v, void* out,
                                int B, int T, int g_q, int g_kv, int d, float scale, gqa_dtype dtype,
                                void* stream);

/*
 * kv_meanpool_heads - MHA -> GQA checkpoint conversion of one projection.
 *
 * GQA paper section 2.1 (Figure 1) and section 2.2; tutorial section 4.3,
 * step 2: each group's key (or value) projection is the mean of the
 * projections of the heads in that group.  Call it once for the key weights
 * and once for the value weights.
 *
 *   w_in   [H, per_head_elems]   dtype, device: head h's weights, contiguous
 *                                (e.g. a [d_model, d_head] matrix per head)
 *   w_out  [G, per_head_elems]   dtype, device:
 *          w_out[g, e] = (sum_{k < n_rep} w_in[g*n_rep + k, e]) / n_rep
 *          summed in float32, divided once (correctly rounded) and rounded
 *          once to dtype.
 *
 * Errors: GQA_ERR_INVALID_ARG for H, G < 1, H % G != 0, per_head_elems < 0,
 * NULL/misaligned pointers (with per_head_elems > 0) or an unknown dtype.
 * per_head_elems = 0 is a valid no-op.
 */
gqa_status kv_meanpool_heads(const void* w_in, void* w_out, int H, int G,
                             int64_t per_head_elems, gqa_dtype dtype, void* stream);

/*
 * kv_meanpool_heads_batch - kv_meanpool_heads over up to
 * GQA_MEANPOOL_MAX_BATCH projections of one shape in a single launch (e.g. the
 * key and value projections of one or several layers, as a checkpoint
 * conversion needs them): projection j reads w_in[j] and writes w_out[j],
 * with exactly the arithmetic and results of kv_meanpool_heads on that pair;
 * one launch pays the fixed cost once.
 *
 *   w_in, w_out  host arrays of `count` device pointers (the arrays are read
 *                during the call only; the pointed-to tensors must not
 *                overlap between an input and any output)
 *   count        0 .. GQA_MEANPOOL_MAX_BATCH (0: a valid no-op)
 *
 * Errors: as kv_meanpool_heads, plus GQA_ERR_INVALID_ARG for a count out of
 * range, a NULL array or a NULL/misaligned pointer in it.
 */
#define GQA_MEANPOOL_MAX_BATCH 16
gqa_status kv_meanpool_heads_batch(const void* const* w_in, void* const* w_out, int count, int H,
                                   int G, int64_t per_head_elems, gqa_dtype dtype, void* stream);

/*
 * gqa_decode_noalloc - gqa_decode_split for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, kernels and results, with the
 * split partials and arrival counters in a static device array of
 * GQA_NOALLOC_SCRATCH_BYTES inside the library instead of a caller workspace.
 *
 * The caller still passes every input and output (same meaning, layout and
 * checks as gqa_decode_split).  The call itself allocates nothing
 * (no hipMalloc/hipFree or allocating library routine).  The array exists once
 * per GPU the library runs on, for the life of the process; the first call on
 * a device looks up its address there (hipGetSymbolAddress, on the current
 * device: `stream` must belong to it) and enqueues one small kernel on
 * `stream` that clears the counter header.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that may overlap in time on one GPU (other streams, other
 * threads) RACE and must be serialised by the caller.
 *
 * Errors: as gqa_decode_split; GQA_ERR_WORKSPACE when the shape's split
 * partials (gqa_decode_workspace_bytes with the same arguments) exceed
 * GQA_NOALLOC_SCRATCH_BYTES -- e.g. the planner's split of 64 sequences x 32
 * heads x d=128 over 32768 positions needs about 12 MB and fits; lower
 * num_splits to fit larger batches.  GQA_ERR_LAUNCH if the set-up fails.
 */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
gqa_status gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seqlens, void* out,
                              int B, int H, int G, int d, int n_max, float scale, gqa_dtype dtype,
                              int num_splits, void* stream);

/* Static text for a status code ("GQA_OK", ...); never NULL. */
const char* gqa_status_string(int status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* gqa_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int gqa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
