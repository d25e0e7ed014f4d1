// C ABI of libgqa.so: argument checks, split planning and kernel dispatch.
//
// Everything here runs on the host.  Invalid calls are rejected before any
// HIP runtime call, so the checks can be exercised on a machine without a GPU.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/gqa.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

#ifdef GQA_DECODE_TIMELINE
// Measurement build only (libgqa_timeline.so): where the matrix-core decode
// kernel writes its per-workgroup phase timestamps.
uint64_t* g_timeline = nullptr;
#endif

gqa_status fail(gqa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gqa_status ok() { return GQA_OK; }

bool known_dtype(int dtype) {
  return dtype == GQA_DTYPE_F32 || dtype == GQA_DTYPE_BF16 || dtype == GQA_DTYPE_F16;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split planning.  The decode kernels run one workgroup per (sequence,
// K/V head, split) -- per 16 queries of the head when a group has 32 or more
// (split_units).  A grid of 128 or more work groups runs unsplit: there the
// merge of the partial results (written, acknowledged, counted and read back)
// costs more than a wider grid gains (the Llama-7B-sized G=8 step, 128 work
// groups: 14.7 us unsplit, 15.1 with 2 splits, 16.6 with 3).  Smaller grids
// are split to about 192 work groups in all (G=4, 64 work groups: 3 splits
// 10.7 us, 4 11.0, 2 11.2, 6 12.3; G=1, 32 work groups: 4 splits 9.0 us, 3
// 9.5, 6 9.6, 8 9.8, 2 10.4).
// Splits are whole 32-position tiles and at least 256 positions long, which
// bounds the merge work per position; long caches are cut into slices of at
// most 3072 positions so that ragged lengths balance across the machine (on
// the 64-sequence ragged 32k step, 11 splits of 2979 positions measured ~2%
// faster than 16 of 2048 and than 8, 6 or 4).
constexpr int64_t kUnsplitGrid = 128;
constexpr int64_t kSplitTarget = 192;
constexpr int64_t kMinSplitLen = 256;
constexpr int64_t kMaxSplitLen = 3072;

bool decode_shape_valid(int B, int H, int G, int d, int n_max) {
  if (B < 0 || n_max < 0 || d < 1) return false;
  if (B == 0) return true;
  if (H < 1 || G < 1 || H % G != 0) return false;
  return true;
}

// Work groups per split: one per (sequence, K/V head), times n_rep / 16 when
// a group of 32 or more queries runs as work groups of 16 (as decode_impl
// launches it; GQKVA pairs never do).
int64_t split_units(int B, int H, int G, bool gqkva) {
  const int n_rep = gqkva ? H : H / G;
  const int64_t kv_div = (!gqkva && n_rep > 16 && n_rep % 16 == 0) ? n_rep / 16 : 1;
  return int64_t(B) * G * kv_div;
}

int plan_splits(int64_t units, int n_max) {
  if (units <= 0 || n_max <= 0) return 1;
  int64_t s = units >= kUnsplitGrid ? 1 : ceil_div(kSplitTarget, units);
  s = std::max<int64_t>(s, ceil_div(n_max, kMaxSplitLen));
  s = std::min<int64_t>(s, std::max<int64_t>(1, ceil_div(n_max, kMinSplitLen)));
  // round the slice length to whole 32-position tiles
  int64_t len = ceil_div(ceil_div(n_max, s), 32) * 32;
  return int(ceil_div(n_max, len));
}

// Splits are whole 32-position tiles except possibly the last; the count
// actually used for a requested count S.
void split_geometry(int n_max, int S, int* S_used, int* split_len) {
  if (n_max <= 0 || S <= 1) {
    *S_used = 1;
    *split_len = std::max(n_max, 1);
    return;
  }
  int64_t len = ceil_div(n_max, S);
  if (len >= 32) len = ceil_div(len, 32) * 32;
  *split_len = int(len);
  *S_used = int(ceil_div(n_max, len));
}

// Workspace layout (only when S > 1):
//   [0, 64 KiB)              split-arrival counters, one int per (b, g); every
//                            completed call leaves them zero
//   [64 KiB, +o_bytes)       partial outputs, float [B, H, S, d]
//   [.., +ml_bytes)          partial (max, sum), float [B, H, S, 2]
constexpr size_t kCounterBytes = 65536;
constexpr int64_t kMaxCountedUnits = int64_t(kCounterBytes / sizeof(int));

size_t partial_o_bytes(int B, int H, int d, int S) {
  return size_t(B) * size_t(H) * size_t(S) * size_t(d) * sizeof(float);
}

size_t workspace_for(int B, int H, int d, int S) {
  if (S <= 1 || B <= 0) return 0;
  const size_t o_bytes = partial_o_bytes(B, H, d, S);
  const size_t ml_bytes = size_t(B) * size_t(H) * size_t(S) * 2 * sizeof(float);
  return kCounterBytes + ((o_bytes + 255) / 256) * 256 + ml_bytes;
}

gqa_status launched(hipError_t e, const char* what) {
  if (e == gqa::kAbiMismatch)
    return fail(GQA_ERR_LAUNCH,
                "%s: launch refused: the kernel object and the API object of this library were "
                "built from different versions of the argument structures (rebuild libgqa.so)",
                what);
  if (e != hipSuccess)
    return fail(GQA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// H query heads (GQA) or, with gqkva, H = g_q query groups paired with every
// one of the G K/V groups (H*G outputs).
gqa_status decode_impl(const void* q, const void* k, const void* v, const int32_t* seqlens,
                       void* out, int B, int H, int G, int d, int n_max, float scale, int dtype,
                       int num_splits, void* ws, size_t ws_bytes, void* stream_v,
                       const void* k_new = nullptr, const void* v_new = nullptr,
                       bool gqkva = false, bool check_only = false) {
  g_last_error.clear();
  const bool append = k_new != nullptr || v_new != nullptr;
  if (!known_dtype(dtype)) return fail(GQA_ERR_INVALID_ARG, "gqa_decode: unknown dtype %d", dtype);
  if (B < 0 || n_max < 0)
    return fail(GQA_ERR_INVALID_ARG, "gqa_decode: negative size (B=%d, n_max=%d)", B, n_max);
  if (B == 0) return ok();
  if (H < 1 || G < 1)
    return fail(GQA_ERR_INVALID_ARG, "gqa_decode: H=%d and G=%d must be >= 1", H, G);
  if (!gqkva && H % G != 0)
    return fail(GQA_ERR_INVALID_ARG, "gqa_decode: H=%d is not a multiple of G=%d", H, G);
  if (d < 1) return fail(GQA_ERR_INVALID_ARG, "gqa_decode: head size d=%d", d);
  if (gqkva && int64_t(H) * G > (int64_t(1) << 20))
    return fail(GQA_ERR_INVALID_ARG, "gqkva_decode: too many query x K/V groups");
  // n_rep queries per K/V head; Hp = G * n_rep rows of partial results per sequence
  const int n_rep = gqkva ? H : H / G;
  const int Hp = G * n_rep;
  const gqa::HeadMap hm = gqkva ? gqa::gqkva_head_map(H, G) : gqa::gqa_head_map(G, n_rep);
  if (!std::isfinite(scale)) return fail(GQA_ERR_INVALID_ARG, "gqa_decode: scale is not finite");
  if (num_splits < 0) return fail(GQA_ERR_INVALID_ARG, "gqa_decode: num_splits=%d", num_splits);
  if (!q || !out || !seqlens || (n_max > 0 && (!k || !v)) || (append && (!k_new || !v_new)))
    return fail(GQA_ERR_INVALID_ARG, "gqa_decode: NULL tensor pointer");
  if (append && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(GQA_ERR_INVALID_ARG, "gqa_decode: tensors must be 16-byte aligned");
  if (!aligned16(q) || !aligned16(out) || (n_max > 0 && (!aligned16(k) || !aligned16(v))) ||
      (reinterpret_cast<uintptr_t>(seqlens) & 3u))
    return fail(GQA_ERR_INVALID_ARG, "gqa_decode: tensors must be 16-byte aligned");
  if (d != 64 && d != 128)
    return fail(GQA_ERR_UNSUPPORTED, "gqa_decode: head size d=%d (built for 64 and 128)", d);
  const int64_t n_rows64 = int64_t(B) * Hp;
  if (n_rows64 * d > (int64_t(1) << 40) || int64_t(B) * G * n_max > (int64_t(1) << 40))
    return fail(GQA_ERR_INVALID_ARG, "gqa_decode: problem too large");

  int S_req = num_splits == 0 ? plan_splits(split_units(B, H, G, gqkva), n_max)
                               : std::min(num_splits, std::max(n_max, 1));
  int S, split_len;
  split_geometry(n_max, S_req, &S, &split_len);
  const size_t need = workspace_for(B, Hp, d, S);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws)))
    return fail(GQA_ERR_WORKSPACE, "gqa_decode: workspace of %zu bytes needed, %zu given%s", need,
                ws_bytes, (ws && !aligned16(ws)) ? " (misaligned)" : "");

  if (check_only) return ok();

  float* part_o = nullptr;
  float* part_ml = nullptr;
  int* counters = nullptr;
  if (need > 0) {
    char* base = static_cast<char*>(ws);
    counters = reinterpret_cast<int*>(base);
    part_o = reinterpret_cast<float*>(base + kCounterBytes);
    const size_t o_bytes = partial_o_bytes(B, Hp, d, S);
    part_ml = reinterpret_cast<float*>(base + kCounterBytes + ((o_bytes + 255) / 256) * 256);
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_v);

  // A group of more than 16 queries (one matrix-core tile of heads) runs as
  // several work groups of 16 that read the same K/V head: twice the
  // workgroups for n_rep = 32, each with a single tile of heads; the second
  // read of a K/V slice mostly comes from the last-level cache.
  int kv_div = 1;
  if (!gqkva && n_rep > 16 && n_rep % 16 == 0 && int64_t(B) * G * (n_rep / 16) <= kMaxCountedUnits)
    kv_div = n_rep / 16;
  if (dtype != GQA_DTYPE_F32 && gqa::decode_mfma_supports(n_rep / kv_div, d, S, split_len)) {
    auto p = gqa::problem_for<gqa::DecodeProblem>();
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.seqlens = seqlens;
    p.out = static_cast<uint16_t*>(out);
    p.part_o = part_o;
    p.part_ml = part_ml;
    // the split merge runs inside the decode kernel when the counters fit
    p.counters = (S > 1 && int64_t(B) * G * kv_div <= kMaxCountedUnits) ? counters : nullptr;
    p.k_new = static_cast<const uint16_t*>(k_new);
    p.v_new = static_cast<const uint16_t*>(v_new);
    p.dtype = dtype;
    p.hm = kv_div > 1 ? gqa::gqa_head_map(G * kv_div, n_rep / kv_div) : hm;
    p.B = B; p.H = Hp; p.G = G * kv_div; p.n_rep = n_rep / kv_div; p.d = d; p.n_max = n_max;
    p.kv_div = kv_div;
    p.scale = scale;
    p.num_splits = S;
    p.split_len = split_len;
#ifdef GQA_DECODE_TIMELINE
    p.timeline = g_timeline;
#endif
    gqa_status st = launched(gqa::launch_decode_mfma(p, stream), "gqa_decode");
    if (st != GQA_OK || S == 1 || p.counters != nullptr) return st;
  } else {
    if (append && n_max > 0) {
      // float32 path: the new rows go in first (same stream, so the decode sees them)
      auto a = gqa::problem_for<gqa::AppendProblem>();
      a.k_new = k_new; a.v_new = v_new; a.k = const_cast<void*>(k); a.v = const_cast<void*>(v);
      a.seqlens = seqlens; a.B = B; a.G = G; a.n_max = n_max;
      a.row_bytes = d * (dtype == GQA_DTYPE_F32 ? 4 : 2);
      gqa_status st = launched(gqa::launch_append(a, stream), "gqa_decode_append (append)");
      if (st != GQA_OK) return st;
    }
    auto p = gqa::problem_for<gqa::RowsProblem>();
    p.q = q; p.k = k; p.v = v; p.seqlens = seqlens; p.out = out;
    p.part_o = part_o; p.part_ml = part_ml;
    p.n_rows = B; p.rows_per_batch = 1;
    p.H = Hp; p.G = G; p.n_rep = n_rep; p.d = d;
    p.hm = hm;
    p.kv_batch_stride = int64_t(G) * n_max * d;
    p.kv_group_stride = int64_t(n_max) * d;
    p.kv_pos_stride = d;
    p.n_max = n_max;
    p.causal = 0;
    p.scale = scale;
    p.num_splits = S;
    p.split_len = split_len;
    gqa_status st = launched(gqa::launch_rows_valu(p, dtype, stream), "gqa_decode");
    if (st != GQA_OK) return st;
  }
  if (S > 1) {
    auto c = gqa::problem_for<gqa::CombineProblem>();
    c.part_o = part_o; c.part_ml = part_ml; c.out = out;
    c.n_rows = B; c.H = Hp; c.d = d; c.num_splits = S; c.dtype = dtype;
    c.n_rep = n_rep; c.hm = hm;
    return launched(gqa::launch_combine(c, stream), "gqa_decode (combine)");
  }
  return ok();
}

// Causal attention of T query rows per sequence.  Prompt layout (kv_cap = T,
// K/V [B, T, G, d], ctx_lens null) or cache layout (K/V [B, G, n_max, d],
// row t at position ctx_lens[b] + t).  gqkva: H query groups x G K/V groups.
gqa_status prefill_impl(const char* name, const void* q, const void* k, const void* v, void* out,
                        const int32_t* ctx_lens, bool cache_layout, int B, int T, int H, int G,
                        int d, int n_max, float scale, int dtype, void* stream_v, bool gqkva) {
  g_last_error.clear();
  if (!known_dtype(dtype)) return fail(GQA_ERR_INVALID_ARG, "%s: unknown dtype %d", name, dtype);
  if (B < 0 || T < 0 || n_max < 0)
    return fail(GQA_ERR_INVALID_ARG, "%s: negative size (B=%d, T=%d, n_max=%d)", name, B, T, n_max);
  if (B == 0 || T == 0) return ok();
  if (H < 1 || G < 1) return fail(GQA_ERR_INVALID_ARG, "%s: H=%d and G=%d must be >= 1", name, H, G);
  if (!gqkva && H % G != 0)
    return fail(GQA_ERR_INVALID_ARG, "%s: H=%d is not a multiple of G=%d", name, H, G);
  if (cache_layout && n_max < 1)
    return fail(GQA_ERR_INVALID_ARG, "%s: n_max=%d leaves no room for the chunk", name, n_max);
  if (d < 1) return fail(GQA_ERR_INVALID_ARG, "%s: head size d=%d", name, d);
  if (!std::isfinite(scale)) return fail(GQA_ERR_INVALID_ARG, "%s: scale is not finite", name);
  if (!q || !k || !v || !out || (cache_layout && !ctx_lens))
    return fail(GQA_ERR_INVALID_ARG, "%s: NULL tensor", name);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(ctx_lens) & 3u))
    return fail(GQA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", name);
  if (d != 64 && d != 128)
    return fail(GQA_ERR_UNSUPPORTED, "%s: head size d=%d (built for 64 and 128)", name, d);
  const int n_rep = gqkva ? H : H / G;
  const int64_t out_heads = int64_t(G) * n_rep;
  // (query rows are counted in 32 bits: B*T below 2^31)
  if (int64_t(B) * T * out_heads * d > (int64_t(1) << 40) || int64_t(B) * T > INT32_MAX ||
      (cache_layout && int64_t(B) * G * n_max * d > (int64_t(1) << 40)))
    return fail(GQA_ERR_INVALID_ARG, "%s: problem too large", name);
  const gqa::HeadMap hm = gqkva ? gqa::gqkva_head_map(H, G) : gqa::gqa_head_map(G, n_rep);
  const int kv_cap = cache_layout ? n_max : T;
  const int64_t kv_b = cache_layout ? int64_t(G) * n_max * d : int64_t(T) * G * d;
  const int64_t kv_g = cache_layout ? int64_t(n_max) * d : d;
  const int64_t kv_p = cache_layout ? d : int64_t(G) * d;
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  if (dtype != GQA_DTYPE_F32 && gqa::prefill_mfma_supports(n_rep, d, kv_cap, kv_p)) {
    auto p = gqa::problem_for<gqa::PrefillProblem>();
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.out = static_cast<uint16_t*>(out);
    p.ctx_lens = ctx_lens;
    p.dtype = dtype;
    p.hm = hm;
    p.kv_bstride = kv_b; p.kv_gstride = kv_g; p.kv_pstride = kv_p;
    p.kv_cap = kv_cap;
    p.B = B; p.T = T; p.G = G; p.n_rep = n_rep; p.d = d;
    p.scale = scale;
    return launched(gqa::launch_prefill_mfma(p, stream), name);
  }
  auto p = gqa::problem_for<gqa::RowsProblem>();
  p.q = q; p.k = k; p.v = v; p.seqlens = nullptr; p.out = out;
  p.n_rows = B * T; p.rows_per_batch = T;
  p.H = int(out_heads); p.G = G; p.n_rep = n_rep; p.d = d;
  p.hm = hm;
  p.ctx_lens = ctx_lens;
  p.kv_batch_stride = kv_b;
  p.kv_group_stride = kv_g;
  p.kv_pos_stride = kv_p;
  p.n_max = kv_cap;
  p.causal = 1;
  p.scale = scale;
  p.num_splits = 1;
  p.split_len = kv_cap;
  return launched(gqa::launch_rows_valu(p, dtype, stream), name);
}

// ---------------------------------------------------------------------------
// Decode without allocation: the split workspace lives in a static device
// array (one copy per GPU, held until the process ends) instead of a caller
// buffer.  In host code `scratch` names a host-side stand-in, never the device
// memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is passed on.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = GQA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

// Clears the split-arrival counters (an ordinary kernel: safe under graph
// capture, unlike a memset node).
__global__ void clear_counters_kernel(int* counters, int n) {
  for (int i = int(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += int(gridDim.x * blockDim.x))
    counters[i] = 0;
}

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (set up on the first call
// there: the lookup, then a clear of the counter header enqueued on `stream`,
// ahead of that call's kernels; static storage also starts zeroed).
gqa_status scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQA_ERR_LAUNCH, "gqa_decode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GQA_ERR_UNSUPPORTED, "gqa_decode_noalloc: device %d (at most %d devices)", dev, kMaxDevices);
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    void* ptr = nullptr;
    slot.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (slot.err != hipSuccess) return;
    hipLaunchKernelGGL(clear_counters_kernel, dim3(16), dim3(256), 0, stream, static_cast<int*>(ptr),
                       int(kCounterBytes / sizeof(int)));
    slot.err = hipGetLastError();
    if (slot.err == hipSuccess) slot.ptr = ptr;
  });
  if (slot.err != hipSuccess || slot.ptr == nullptr)
    return fail(GQA_ERR_LAUNCH, "gqa_decode_noalloc: static scratch set-up on device %d failed: %s", dev,
                hipGetErrorString(slot.err));
  *out = slot.ptr;
  return ok();
}

}  // namespace

extern "C" {

int gqa_decode_num_splits(int B, int H, int G, int d, int n_max) {
  if (!decode_shape_valid(B, H, G, d, n_max)) return 0;
  int S, len;
  split_geometry(n_max, plan_splits(split_units(B, H, G, false), n_max), &S, &len);
  return S;
}

size_t gqa_decode_workspace_bytes(int B, int H, int G, int d, int n_max, int num_splits) {
  if (!decode_shape_valid(B, H, G, d, n_max) || num_splits < 0) return size_t(-1);
  int S_req = num_splits == 0 ? plan_splits(split_units(B, H, G, false), n_max)
                               : std::min(num_splits, std::max(n_max, 1));
  int S, len;
  split_geometry(n_max, S_req, &S, &len);
  return workspace_for(B, H, d, S);
}

gqa_status gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seqlens, void* out, int B, int H, int G, int d, int n_max,
                      float scale, gqa_dtype dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode_impl(q, k_cache, v_cache, seqlens, out, B, H, G, d, n_max, scale, dtype, 0,
                     workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_split(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seqlens, void* out, int B, int H, int G, int d,
                            int n_max, float scale, gqa_dtype dtype, int num_splits, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, seqlens, out, B, H, G, d, n_max, scale, dtype,
                     num_splits, workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                             void* v_cache, const int32_t* seqlens, void* out, int B, int H, int G,
                             int d, int n_max, float scale, gqa_dtype dtype, int num_splits,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && (!k_new || !v_new)) {
    g_last_error.clear();
    return fail(GQA_ERR_INVALID_ARG, "gqa_decode_append: NULL k_new / v_new");
  }
  return decode_impl(q, k_cache, v_cache, seqlens, out, B, H, G, d, n_max, scale, dtype,
                     num_splits, workspace, workspace_bytes, stream, k_new, v_new);
}

gqa_status gqa_prefill_causal(const void* q, const void* k, const void* v, void* out, int B,
                              int T, int H, int G, int d, float scale, gqa_dtype dtype, void* stream) {
  return prefill_impl("gqa_prefill_causal", q, k, v, out, nullptr, false, B, T, H, G, d, 0, scale,
                      dtype, stream, false);
}

gqa_status gqa_prefill_chunk(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* ctx_lens, void* out, int B, int T, int H, int G, int d,
                             int n_max, float scale, gqa_dtype dtype, void* stream) {
  return prefill_impl("gqa_prefill_chunk", q, k_cache, v_cache, out, ctx_lens, true, B, T, H, G, d,
                      n_max, scale, dtype, stream, false);
}

gqa_status gqkva_prefill_causal(const void* q, const void* k, const void* v, void* out, int B,
                                int T, int g_q, int g_kv, int d, float scale, gqa_dtype dtype,
                                void* stream) {
  return prefill_impl("gqkva_prefill_causal", q, k, v, out, nullptr, false, B, T, g_q, g_kv, d, 0,
                      scale, dtype, stream, true);
}

gqa_status gqkva_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens, void* out, int B, int g_q, int g_kv, int d,
                        int n_max, float scale, gqa_dtype dtype, int num_splits, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, seqlens, out, B, g_q, g_kv, d, n_max, scale, dtype,
                     num_splits, workspace, workspace_bytes, stream, nullptr, nullptr, true);
}

size_t gqkva_decode_workspace_bytes(int B, int g_q, int g_kv, int d, int n_max, int num_splits) {
  if (B < 0 || n_max < 0 || d < 1 || num_splits < 0 || g_q < 1 || g_kv < 1) return size_t(-1);
  int S_req = num_splits == 0 ? plan_splits(split_units(B, g_q, g_kv, true), n_max)
                               : std::min(num_splits, std::max(n_max, 1));
  int S, len;
  split_geometry(n_max, S_req, &S, &len);
  return workspace_for(B, g_q * g_kv, d, S);
}

static_assert(gqa::kMaxMeanpoolBatch == GQA_MEANPOOL_MAX_BATCH, "one batch limit");

gqa_status kv_meanpool_heads_batch(const void* const* w_in, void* const* w_out, int count, int H, int G,
                                   int64_t per_head_elems, gqa_dtype dtype, void* stream_v) {
  g_last_error.clear();
  if (!known_dtype(dtype))
    return fail(GQA_ERR_INVALID_ARG, "kv_meanpool_heads: unknown dtype %d", dtype);
  if (count < 0 || count > GQA_MEANPOOL_MAX_BATCH)
    return fail(GQA_ERR_INVALID_ARG, "kv_meanpool_heads_batch: count=%d (0 .. %d)", count,
                GQA_MEANPOOL_MAX_BATCH);
  if (H < 1 || G < 1 || H % G != 0)
    return fail(GQA_ERR_INVALID_ARG, "kv_meanpool_heads: H=%d must be a positive multiple of G=%d",
                H, G);
  if (per_head_elems < 0)
    return fail(GQA_ERR_INVALID_ARG, "kv_meanpool_heads: per_head_elems=%lld",
                (long long)per_head_elems);
  if (per_head_elems == 0 || count == 0) return ok();
  if (!w_in || !w_out) return fail(GQA_ERR_INVALID_ARG, "kv_meanpool_heads_batch: NULL pointer array");
  for (int j = 0; j < count; ++j) {
    if (!w_in[j] || !w_out[j]) return fail(GQA_ERR_INVALID_ARG, "kv_meanpool_heads: NULL tensor (projection %d)", j);
    if (!aligned16(w_in[j]) || !aligned16(w_out[j]))
      return fail(GQA_ERR_INVALID_ARG, "kv_meanpool_heads: tensors must be 16-byte aligned (projection %d)", j);
  }
  if (int64_t(H) * per_head_elems > (int64_t(1) << 40))
    return fail(GQA_ERR_INVALID_ARG, "kv_meanpool_heads: problem too large");
  auto p = gqa::problem_for<gqa::MeanpoolProblem>();
  for (int j = 0; j < gqa::kMaxMeanpoolBatch; ++j) {
    p.w_in[j] = j < count ? w_in[j] : nullptr;
    p.w_out[j] = j < count ? w_out[j] : nullptr;
  }
  p.count = count;
  p.H = H; p.G = G; p.n_rep = H / G;
  p.per_head_elems = per_head_elems; p.dtype = dtype;
  return launched(gqa::launch_meanpool(p, static_cast<hipStream_t>(stream_v)),
                  "kv_meanpool_heads");
}

gqa_status kv_meanpool_heads(const void* w_in, void* w_out, int H, int G, int64_t per_head_elems,
                             gqa_dtype dtype, void* stream_v) {
  return kv_meanpool_heads_batch(&w_in, &w_out, 1, H, G, per_head_elems, dtype, stream_v);
}

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARG: return "GQA_ERR_INVALID_ARG";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE";
    case GQA_ERR_LAUNCH: return "GQA_ERR_LAUNCH";
    default: return "GQA_ERR_UNKNOWN";
  }
}

const char* gqa_last_error(void) { return g_last_error.c_str(); }

int gqa_version(void) { return 100; }

#ifdef GQA_DECODE_TIMELINE
// Measurement build only: device buffer of 8 uint64 per workgroup of the next
// matrix-core decode launches (NULL: none recorded).
void gqa_timeline_set_buffer(uint64_t* buf) { g_timeline = buf; }
#endif

gqa_status gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seqlens, void* out, int B, int H, int G, int d,
                              int n_max, float scale, gqa_dtype dtype, int num_splits,
                              void* stream) {
  g_last_error.clear();
  if (!decode_shape_valid(B, H, G, d, n_max) || num_splits < 0)
    // the full argument checks (with their messages) are decode_impl's
    return decode_impl(q, k_cache, v_cache, seqlens, out, B, H, G, d, n_max, scale, dtype,
                       num_splits, nullptr, 0, stream);
  int S_req = B == 0 ? 1
                     : (num_splits == 0 ? plan_splits(split_units(B, H, G, false), n_max)
                                        : std::min(num_splits, std::max(n_max, 1)));
  int S, len;
  split_geometry(n_max, S_req, &S, &len);
  const size_t need = workspace_for(B, H, d, S);
  if (need > kScratchBytes)
    return fail(GQA_ERR_WORKSPACE,
                "gqa_decode_noalloc: this shape needs %zu bytes of split scratch (B=%d, H=%d, d=%d, "
                "%d splits); the static scratch holds %zu (GQA_NOALLOC_SCRATCH_BYTES): use "
                "gqa_decode_split with a workspace, or fewer splits",
                need, B, H, d, S, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    // argument errors first, so that an invalid call makes no HIP call
    gqa_status st = decode_impl(q, k_cache, v_cache, seqlens, out, B, H, G, d, n_max, scale,
                                dtype, num_splits, reinterpret_cast<void*>(uintptr_t(256)),
                                kScratchBytes, stream, nullptr, nullptr, false, /*check_only=*/true);
    if (st != GQA_OK) return st;
    st = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws);
    if (st != GQA_OK) return st;
  }
  return decode_impl(q, k_cache, v_cache, seqlens, out, B, H, G, d, n_max, scale, dtype,
                     num_splits, ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
