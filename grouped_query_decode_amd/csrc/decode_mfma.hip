// GQA decode step on the gfx950 matrix cores (bfloat16 in, float32 accumulate).
//
// Definition: fogdragon CSDN blog, section "KV Cache" (append, then
// softmax(scale * q.K) over the cached positions and a weighted sum of V);
// GQA paper section 2.2 (n_rep = H/G query heads share one K/V head).
//
// Work unit: one workgroup of 1, 2 or 4 waves per (sequence b, K/V head g,
// split s).  The group's n_rep query heads are the 16 columns of the
// matrix-core tiles (padded with zero queries), so every cached K/V row is read
// from HBM once and used by all heads of its group:
//
//   scores  S^T[key][head] = K[key][:] . Q[head][:]     16x16x32 bf16 MFMA,
//           A = 16 keys x 32 dims straight from HBM (16-byte loads),
//           B = the group's queries (registers, loaded once)
//   softmax online, base 2 (hardware exp2), float32; the weights are rounded to bf16 and the
//           normaliser sums the rounded weights (so constant V is exact)
//   output  O^T[dim][head] += V^T[dim][key] P^T[key][head]   16x16x32 MFMA,
//           A = V^T gathered from a per-wave LDS copy of the 32-row V tile,
//           B = the weights, already in the right lanes after the scores
//
// Each wave walks its own 32-position tiles of the split (tile t goes to wave
// t mod waves) with a one-tile register prefetch; the waves merge (max, sum,
// output) through LDS.  With several splits, each workgroup writes its
// partial (max, sum, output) per head; the last workgroup of a (b, g) to
// finish -- found with a counter in the workspace header, which it resets --
// merges the partials (log-sum-exp) and writes the output, so one launch does
// the whole step.  Positions at or beyond the sequence length are never
// loaded: their K rows are zero, their scores are set to -inf before the
// softmax and their V rows are zero, so cache contents there (NaN included)
// cannot reach the arithmetic.

#include "device_common.h"
#include "internal.h"

namespace gqa {
namespace {

constexpr int kKT = 32;        // positions per wave step
constexpr int kMaxWaves = 4;

template <int D>
struct Cfg {
  static constexpr int kSteps = D / 32;           // MFMA k-steps over the head dimension
  static constexpr int kColBlocks = D / 16;       // 16-wide output column blocks
  static constexpr int kChunks = D / 8;           // 16-byte chunks per cached row
  static constexpr int kVLoads = kKT * kChunks / 64;
  static constexpr int kPitch = D * 2 + 16;       // LDS bytes per V row (bank spread)
  static constexpr int kWaveLds = kKT * kPitch;
  static constexpr int kMergeRow = D + 4;         // floats per head row in the merge area
  static constexpr int kMergeBytes = (kMaxWaves * 16 * kMergeRow + 3 * kMaxWaves * 16 + 32) * 4;
  static constexpr int kLds = kMaxWaves * kWaveLds > kMergeBytes ? kMaxWaves * kWaveLds : kMergeBytes;
};

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Partials cross workgroups (and XCDs, whose L2s are not coherent with each
// other).  They are written and read with buffer instructions carrying the
// device-coherence bit (sc1) -- the same access an agent-scope relaxed atomic
// makes, but 16 bytes wide and free to overlap -- so no device-wide cache
// writeback or invalidate is needed.  A buffer load past the end of its
// resource returns zeros.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kDeviceCoherent = 16;    // cache-policy bit sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Log-sum-exp merge of the S split partials of NI (head, 8-column chunk)
// items of sequence b, written to out.  Splits are read 8 at a time with all
// their loads (for every item) in flight together; the running maximum is
// rescaled per batch.
template <int D, int NI>
__device__ __forceinline__ void merge_items(const DecodeProblem& p, int b, const int* hs, const int* c8s) {
  const int S = p.num_splits;
  __amdgpu_buffer_rsrc_t rml[NI], ro[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t pr0 = (int64_t(b) * p.H + hs[i]) * S;
    rml[i] = rsrc(p.part_ml + pr0 * 2, uint32_t(S) * 8u);
    ro[i] = rsrc(p.part_o + pr0 * D, uint32_t(S) * D * 4u);
  }
  float M[NI], L[NI], O[NI][8];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    M[i] = -INFINITY;
    L[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) O[i][e] = 0.f;
  }
  for (int s0 = 0; s0 < S; s0 += 8) {
    u32x2_t ml[NI][8];
    u32x4_t oa[NI][8], ob[NI][8];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + u;                      // s >= S reads zeros (l = 0: skipped)
        ml[i][u] = __builtin_amdgcn_raw_buffer_load_b64(rml[i], s * 8, 0, kDeviceCoherent);
        oa[i][u] = __builtin_amdgcn_raw_buffer_load_b128(ro[i], s * D * 4 + c8s[i] * 32, 0, kDeviceCoherent);
        ob[i][u] = __builtin_amdgcn_raw_buffer_load_b128(ro[i], s * D * 4 + c8s[i] * 32 + 16, 0, kDeviceCoherent);
      }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float cm = M[i];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (__uint_as_float(ml[i][u][1]) > 0.f) cm = fmaxf(cm, __uint_as_float(ml[i][u][0]));
      if (cm == -INFINITY) continue;             // nothing seen yet
      const float f0 = exp2f(M[i] - cm);         // 0 while M is -inf
      L[i] *= f0;
#pragma unroll
      for (int e = 0; e < 8; ++e) O[i][e] *= f0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float lu = __uint_as_float(ml[i][u][1]);
        const float f = lu > 0.f ? exp2f(__uint_as_float(ml[i][u][0]) - cm) : 0.f;
        L[i] = fmaf(lu, f, L[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          O[i][e] = fmaf(__uint_as_float(oa[i][u][e]), f, O[i][e]);
          O[i][4 + e] = fmaf(__uint_as_float(ob[i][u][e]), f, O[i][4 + e]);
        }
      }
      M[i] = cm;
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float inv = L[i] > 0.f ? 1.f / L[i] : 0.f;
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(O[i][2 * e] * inv, O[i][2 * e + 1] * inv);
    st16(p.out + (int64_t(b) * p.H + hs[i]) * D + c8s[i] * 8, w);
  }
}

template <int D>
__device__ __forceinline__ void merge_splits(const DecodeProblem& p, int b, int h, int c8) {
  merge_items<D, 1>(p, b, &h, &c8);
}

template <int D>
__device__ __forceinline__ void merge_splits2(const DecodeProblem& p, int b, int h0, int c0, int h1, int c1) {
  const int hs[2] = {h0, h1};
  const int cs[2] = {c0, c1};
  merge_items<D, 2>(p, b, hs, cs);
}

template <int D, int NHB>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(DecodeProblem p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::kLds];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int lo = lane & 15;
  const int hi = lane >> 4;

  const int S = p.num_splits;
  const int s = int(blockIdx.x % unsigned(S));
  const int unit = int(blockIdx.x / unsigned(S));
  const int g = unit % p.G;
  const int b = unit / p.G;

  int len = p.seqlens[b];
  len = len < 0 ? 0 : (len > p.n_max ? p.n_max : len);
  const int j0 = s * p.split_len;
  const int j1 = min(len, j0 + p.split_len);

  const int64_t kv_off = (int64_t(b) * p.G + g) * int64_t(p.n_max) * D;
  const uint16_t* kb = p.k + kv_off;
  const uint16_t* vb = p.v + kv_off;

  // Queries of the group: B operand of the score MFMA, lane = head lo of head
  // block hb, k-slot group hi covers dims 8*(4*ks + hi) .. +7.
  bf16x8_t qop[NHB][C::kSteps];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int hl = hb * 16 + lo;
    const bool hv = hl < p.n_rep;
    const uint16_t* qrow = p.q + (int64_t(b) * p.H + g * p.n_rep + (hv ? hl : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < C::kSteps; ++ks) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (hv) w = ld16(qrow + (4 * ks + hi) * 8);
      qop[hb][ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x4_t acc[NHB][C::kColBlocks];
  float mrun[NHB], lrun[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    mrun[hb] = -INFINITY;
    lrun[hb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb) acc[hb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = p.scale * kLog2e;
  char* myv = smem + wave * C::kWaveLds;

  u32x4_t kreg[2][C::kSteps];
  u32x4_t vreg[C::kVLoads];

  auto load_tile = [&](int jt) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int key = jt + 16 * blk + lo;
#pragma unroll
      for (int ks = 0; ks < C::kSteps; ++ks) {
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (key < j1) w = ld16_stream(kb + int64_t(key) * D + (4 * ks + hi) * 8);
        kreg[blk][ks] = w;
      }
    }
#pragma unroll
    for (int t = 0; t < C::kVLoads; ++t) {
      const int idx = t * 64 + lane;
      const int key = jt + idx / C::kChunks;
      const int ch = idx % C::kChunks;
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (key < j1) w = ld16_stream(vb + int64_t(key) * D + ch * 8);
      vreg[t] = w;
    }
  };

  int jt = j0 + wave * kKT;
  if (jt < j1) load_tile(jt);
  for (; jt < j1; jt += nw * kKT) {
    u32x4_t kc[2][C::kSteps];
    u32x4_t vc[C::kVLoads];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int ks = 0; ks < C::kSteps; ++ks) kc[blk][ks] = kreg[blk][ks];
#pragma unroll
    for (int t = 0; t < C::kVLoads; ++t) vc[t] = vreg[t];
    if (jt + nw * kKT < j1) load_tile(jt + nw * kKT);

    // V rows of this tile into the wave's LDS area (row-major, padded rows)
#pragma unroll
    for (int t = 0; t < C::kVLoads; ++t) {
      const int idx = t * 64 + lane;
      const int kl = idx / C::kChunks;
      const int ch = idx % C::kChunks;
      *reinterpret_cast<u32x4_t*>(myv + kl * C::kPitch + ch * 16) = vc[t];
    }

    // scores
    f32x4_t sacc[NHB][2];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::kSteps; ++ks)
          a = mfma16(__builtin_bit_cast(bf16x8_t, kc[blk][ks]), qop[hb][ks], a);
        sacc[hb][blk] = a;
      }

    // online softmax; lane holds keys jt + 16*blk + 4*hi + r of head lo
    bf16x8_t pop[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float t2[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = jt + 16 * blk + 4 * hi + r;
          const float x = key < j1 ? sacc[hb][blk][r] * c2 : -INFINITY;
          t2[blk][r] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const float mn = fmaxf(mrun[hb], tmax);      // finite: position jt is valid
      const float alpha = __builtin_amdgcn_exp2f(mrun[hb] - mn);
      mrun[hb] = mn;
      uint32_t w[4];
      float lsum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          const uint32_t pk = pack_bf16x2(__builtin_amdgcn_exp2f(t2[blk][2 * r2] - mn),
                                          __builtin_amdgcn_exp2f(t2[blk][2 * r2 + 1] - mn));
          w[blk * 2 + r2] = pk;
          lsum += bf16lo_to_f32(pk) + bf16hi_to_f32(pk);
        }
      lrun[hb] = fmaf(lrun[hb], alpha, lsum);
      pop[hb] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]});
#pragma unroll
      for (int cb = 0; cb < C::kColBlocks; ++cb) acc[hb][cb] *= alpha;
    }

    lds_wave_sync();
    // weighted sum of values
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb) {
      const int col = 16 * cb + lo;
      bf16x8_t vop;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kl = 16 * (e >> 2) + 4 * hi + (e & 3);
        vop[e] = __builtin_bit_cast(__bf16, *reinterpret_cast<const uint16_t*>(myv + kl * C::kPitch + col * 2));
      }
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) acc[hb][cb] = mfma16(vop, pop[hb], acc[hb][cb]);
    }
    lds_wave_sync();
  }

  // per-head normaliser: the four lanes of a head hold disjoint positions
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float x = lrun[hb];
    x += shfl_xor(x, 16);
    x += shfl_xor(x, 32);
    lrun[hb] = x;
  }

  // Merge the waves, one head block at a time, and write the output (one
  // split) or this split's partial result.  One thread per head computes the
  // merged maximum, the per-wave factors and the normaliser; then every thread
  // combines 4 output columns of one head.
  float* sm_o = reinterpret_cast<float*>(smem);
  float* sm_m = sm_o + kMaxWaves * 16 * C::kMergeRow;
  float* sm_l = sm_m + kMaxWaves * 16;
  float* sm_f = sm_l + kMaxWaves * 16;
  float* sm_hd = sm_f + kMaxWaves * 16;      // per head: merged max, then normaliser (or 1/it)
  constexpr int kC4 = D / 4;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb)
      *reinterpret_cast<f32x4_t*>(sm_o + (wave * 16 + lo) * C::kMergeRow + 16 * cb + 4 * hi) = acc[hb][cb];
    if (hi == 0) {
      sm_m[wave * 16 + lo] = mrun[hb];
      sm_l[wave * 16 + lo] = lrun[hb];
    }
    __syncthreads();
    if (threadIdx.x < 16) {
      const int hl = threadIdx.x;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kMaxWaves; ++w)
        if (w < nw && sm_l[w * 16 + hl] > 0.f) M = fmaxf(M, sm_m[w * 16 + hl]);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < kMaxWaves; ++w) {
        if (w < nw) {
          const float lw = sm_l[w * 16 + hl];
          const float f = lw > 0.f ? exp2f(sm_m[w * 16 + hl] - M) : 0.f;
          sm_f[w * 16 + hl] = f;
          L = fmaf(lw, f, L);
        }
      }
      sm_hd[hl] = M;
      sm_hd[16 + hl] = S == 1 ? (L > 0.f ? 1.f / L : 0.f) : L;
    }
    __syncthreads();
    const int nh = min(16, p.n_rep - 16 * hb);
    for (int t = threadIdx.x; t < nh * kC4; t += blockDim.x) {
      const int hl = t / kC4;
      const int c4 = t % kC4;
      f32x4_t O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kMaxWaves; ++w)
        if (w < nw) O += sm_f[w * 16 + hl] * *reinterpret_cast<const f32x4_t*>(sm_o + (w * 16 + hl) * C::kMergeRow + c4 * 4);
      const int h = g * p.n_rep + 16 * hb + hl;
      if (S == 1) {
        const float inv = sm_hd[16 + hl];
        *reinterpret_cast<uint2*>(p.out + (int64_t(b) * p.H + h) * D + c4 * 4) =
            make_uint2(pack_bf16x2(O[0] * inv, O[1] * inv), pack_bf16x2(O[2] * inv, O[3] * inv));
      } else {
        const int64_t pr = (int64_t(b) * p.H + h) * S + s;
        const __amdgpu_buffer_rsrc_t ro = rsrc(p.part_o + pr * D, D * 4u);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{__float_as_uint(O[0]), __float_as_uint(O[1]), __float_as_uint(O[2]), __float_as_uint(O[3])},
            ro, c4 * 16, 0, kDeviceCoherent);
        if (c4 == 0) {
          const __amdgpu_buffer_rsrc_t rml = rsrc(p.part_ml + pr * 2, 8u);
          __builtin_amdgcn_raw_buffer_store_b64(
              u32x2_t{__float_as_uint(sm_hd[hl]), __float_as_uint(sm_hd[16 + hl])}, rml, 0, 0, kDeviceCoherent);
        }
      }
    }
  }
  if (S == 1 || p.counters == nullptr) return;

  // Split merge by the last workgroup of this (b, g) to finish.  Each thread
  // waits until its device-coherent partial stores are acknowledged before the
  // workgroup counts itself in; the workgroup that completes the count reads
  // every partial back with device-coherent loads issued after that.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(p.counters + unit, 1);
    s_last = (old == S - 1);
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0)            // ready for the next call (nothing reads it in this one)
    __hip_atomic_store(p.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  constexpr int kC8 = D / 8;
  const int items = p.n_rep * kC8;
  const int t0 = threadIdx.x;
  const int t1 = threadIdx.x + blockDim.x;
  if (t1 < items) {
    merge_splits2<D>(p, b, g * p.n_rep + t0 / kC8, t0 % kC8, g * p.n_rep + t1 / kC8, t1 % kC8);
    for (int t = t1 + blockDim.x; t < items; t += blockDim.x)
      merge_splits<D>(p, b, g * p.n_rep + t / kC8, t % kC8);
  } else if (t0 < items) {
    merge_splits<D>(p, b, g * p.n_rep + t0 / kC8, t0 % kC8);
  }
}

template <int D, int NHB>
hipError_t launch_t(const DecodeProblem& p, hipStream_t stream) {
  const int64_t blocks = int64_t(p.B) * p.G * p.num_splits;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // one wave per 32-position tile of a split, at most four
  const int tiles = (p.split_len + kKT - 1) / kKT;
  const int waves = tiles >= 4 ? 4 : (tiles >= 2 ? 2 : 1);
  hipLaunchKernelGGL((decode_mfma_kernel<D, NHB>), dim3(unsigned(blocks)), dim3(64 * waves), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_supports(int n_rep, int d) {
  return (d == 64 || d == 128) && n_rep >= 1 && n_rep <= 32;
}

hipError_t launch_decode_mfma(const DecodeProblem& p, hipStream_t stream) {
  if (p.d == 128) {
    return p.n_rep <= 16 ? launch_t<128, 1>(p, stream) : launch_t<128, 2>(p, stream);
  }
  return p.n_rep <= 16 ? launch_t<64, 1>(p, stream) : launch_t<64, 2>(p, stream);
}

}  // namespace gqa
