// Internal interface between the C-ABI layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Every problem structure below starts with abi_bytes, the structure's size as
// the code that filled it in saw it; each launcher compares that with its own
// sizeof and refuses the launch (kAbiMismatch, before any HIP call) when they
// differ.  Kernel files and the C-ABI layer are separate objects: a library
// linked from objects built against different versions of this header would
// otherwise hand a kernel shifted arguments.
constexpr hipError_t kAbiMismatch = hipErrorInvalidKernelFile;

template <class P>
inline P problem_for() {
  P p{};
  p.abi_bytes = uint32_t(sizeof(P));
  return p;
}

template <class P>
inline bool abi_ok(const P& p) {
  return p.abi_bytes == uint32_t(sizeof(P));
}

enum Dtype { kF32 = 0, kBF16 = 1, kF16 = 2 };

// Which query row feeds, and which output row receives, query r (0 .. n_rep-1)
// of K/V head g.  GQA: q head g*n_rep + r and the same output head.  GQKVA
// (every query group with every K/V group): q head r, output head r*G + g.
struct HeadMap {
  int q_heads, q_g, q_r;    // q head = g*q_g + r*q_r, q_heads per token row
  int o_heads, o_g, o_r;    // out head = g*o_g + r*o_r, o_heads per token row
  __host__ __device__ int64_t q_head(int g, int r) const { return int64_t(g) * q_g + int64_t(r) * q_r; }
  __host__ __device__ int64_t o_head(int g, int r) const { return int64_t(g) * o_g + int64_t(r) * o_r; }
};

inline HeadMap gqa_head_map(int G, int n_rep) {
  return HeadMap{G * n_rep, n_rep, 1, G * n_rep, n_rep, 1};
}
inline HeadMap gqkva_head_map(int g_q, int g_kv) {
  return HeadMap{g_q, 0, 1, g_q * g_kv, 1, g_kv};
}

// Generic "rows of queries attend a K/V head" problem, used by the vector-unit
// kernel for decode (one row per sequence) and for float32 causal prefill (one
// row per prompt position).  All strides are in elements.
struct RowsProblem {
  uint32_t abi_bytes;        // sizeof(RowsProblem) where it was filled in (see problem_for)
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seqlens;   // decode only (causal == 0)
  void* out;
  float* part_o;            // [rows, H, S, d] float32, when S > 1
  float* part_ml;           // [rows, H, S, 2] (running max, normaliser), when S > 1
  int n_rows;               // decode: B; prefill: B*T
  int rows_per_batch;       // decode: 1; prefill: T
  int H, G, n_rep, d;       // H = G*n_rep (the partial results' layout)
  HeadMap hm;               // q / out rows of (g, r); rows are hm.q_heads*d / hm.o_heads*d apart
  const int32_t* ctx_lens;  // causal: positions before row 0 of each batch (null: none)
  int64_t kv_batch_stride;  // between batches
  int64_t kv_group_stride;  // between K/V heads
  int64_t kv_pos_stride;    // between cached positions
  int n_max;                // decode: cache capacity; prefill: T
  int causal;               // 0: length from seqlens; 1: row i attends 0..ctx+i
  float scale;
  int num_splits;           // S
  int split_len;            // positions per split
};

// Batched decode on the matrix cores (bf16 only).
struct DecodeProblem {
  uint32_t abi_bytes;        // sizeof(DecodeProblem) where it was filled in (see problem_for)
  const uint16_t* q;        // [B, H, d]
  const uint16_t* k;        // [B, G, n_max, d]
  const uint16_t* v;
  const int32_t* seqlens;
  uint16_t* out;            // [B, H, d]
  float* part_o;
  float* part_ml;
  int* counters;            // [B*G] split-arrival counters (zero between calls), or null
  const uint16_t* k_new;    // [B, G, d] this step's k, v to append at seqlens[b]-1, or null
  const uint16_t* v_new;
  int dtype;                // kBF16 or kF16
  HeadMap hm;
  // G work groups of n_rep queries; with kv_div > 1 a K/V head's queries are
  // spread over kv_div consecutive work groups (blocks of n_rep), which all
  // read that head: work group g reads K/V head g / kv_div of G / kv_div.
  int B, H, G, n_rep, d, n_max;   // H = G*n_rep (the partial results' layout)
  int kv_div;
  float scale;
  int num_splits, split_len;
#ifdef GQA_DECODE_TIMELINE
  uint64_t* timeline;       // [grid][8] phase timestamps (the timeline build only)
#endif
};

struct CombineProblem {
  uint32_t abi_bytes;        // sizeof(CombineProblem) where it was filled in (see problem_for)
  const float* part_o;
  const float* part_ml;
  void* out;                // rows of hm.o_heads*d elements, in dtype
  int n_rows, H, d, num_splits;
  int n_rep;                // partial head h = g*n_rep + r goes to out head hm.o_head(g, r)
  HeadMap hm;
  int dtype;
};

// Causal attention of T query rows per sequence on the matrix cores.  Row t
// of sequence b sits at position ctx_b + t (ctx_b = ctx_lens[b], or 0) and
// attends positions 0 .. min(ctx_b + t, kv_cap - 1) of its K/V head.
struct PrefillProblem {
  uint32_t abi_bytes;        // sizeof(PrefillProblem) where it was filled in (see problem_for)
  const uint16_t* q;        // [B, T, hm.q_heads, d]
  const uint16_t* k;        // position j of (b, g) at b*kv_bstride + g*kv_gstride + j*kv_pstride
  const uint16_t* v;
  uint16_t* out;            // [B, T, hm.o_heads, d]
  const int32_t* ctx_lens;  // [B] or null
  int dtype;                // kBF16 or kF16
  HeadMap hm;
  int64_t kv_bstride, kv_gstride, kv_pstride;
  int kv_cap;               // positions that exist per (b, g)
  int B, T, G, n_rep, d;
  float scale;
};

// Write this step's k, v rows into the caches at position seqlens[b]-1
// (when 1 <= seqlens[b] <= n_max), any element type.
struct AppendProblem {
  uint32_t abi_bytes;        // sizeof(AppendProblem) where it was filled in (see problem_for)
  const void* k_new;        // [B, G, row_bytes]
  const void* v_new;
  void* k;                  // [B, G, n_max, row_bytes]
  void* v;
  const int32_t* seqlens;
  int B, G, n_max;
  int row_bytes;            // d * itemsize, a multiple of 16
};

constexpr int kMaxMeanpoolBatch = 16;   // projections per launch (GQA_MEANPOOL_MAX_BATCH)
struct MeanpoolProblem {
  uint32_t abi_bytes;        // sizeof(MeanpoolProblem) where it was filled in (see problem_for)
  const void* w_in[kMaxMeanpoolBatch];   // projection j's input and output (j < count)
  void* w_out[kMaxMeanpoolBatch];
  int count;
  int H, G, n_rep;
  int64_t per_head_elems;
  int dtype;
};

// Launchers: each returns hipSuccess or the launch error.
hipError_t launch_rows_valu(const RowsProblem& p, int dtype, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeProblem& p, hipStream_t stream);
// the split geometry bounds the 32-bit byte offsets of the kernel's buffer accesses
bool decode_mfma_supports(int n_rep, int d, int num_splits, int split_len);
hipError_t launch_combine(const CombineProblem& p, hipStream_t stream);
hipError_t launch_append(const AppendProblem& p, hipStream_t stream);
hipError_t launch_prefill_mfma(const PrefillProblem& p, hipStream_t stream);
bool prefill_mfma_supports(int n_rep, int d, int kv_cap, int64_t kv_pstride);
hipError_t launch_meanpool(const MeanpoolProblem& p, hipStream_t stream);

}  // namespace gqa
