// GQA decode step on the gfx950 matrix cores (bfloat16 in, float32 accumulate).
//
// Definition: fogdragon CSDN blog, section "KV Cache" (append, then
// softmax(scale * q.K) over the cached positions and a weighted sum of V);
// GQA paper section 2.2 (n_rep = H/G query heads share one K/V head).
//
// Work unit: one workgroup of 4 waves per (sequence b, K/V head g, split s).
// The group's n_rep query heads are the 16 columns of the matrix-core tiles
// (padded with zero queries), so every cached K/V row is read from HBM once
// and used by all heads of its group:
//
//   scores  S^T[key][head] = K[key][:] . Q[head][:]     16x16x32 bf16 MFMA,
//           A = 16 keys x 32 dims straight from HBM (16-byte loads),
//           B = the group's queries (registers, loaded once)
//   softmax online, base 2, float32; the weights are rounded to bf16 and the
//           normaliser sums the rounded weights (so constant V is exact)
//   output  O^T[dim][head] += V^T[dim][key] P^T[key][head]   16x16x32 MFMA,
//           A = V^T gathered from a per-wave LDS copy of the 32-row V tile,
//           B = the weights, already in the right lanes after the scores
//
// Each wave walks its own 32-position tiles of the split (tile t goes to wave
// t mod 4) with a one-tile register prefetch; the four waves merge (max, sum,
// output) through LDS at the end.  Positions at or beyond the sequence length
// are never loaded: their K rows are zero, their scores are set to -inf before
// the softmax and their V rows are zero, so cache contents there (NaN included)
// cannot reach the arithmetic.

#include "device_common.h"
#include "internal.h"

namespace gqa {
namespace {

constexpr int kKT = 32;        // positions per wave step
constexpr int kWaves = 4;

template <int D>
struct Cfg {
  static constexpr int kSteps = D / 32;           // MFMA k-steps over the head dimension
  static constexpr int kColBlocks = D / 16;       // 16-wide output column blocks
  static constexpr int kChunks = D / 8;           // 16-byte chunks per cached row
  static constexpr int kVLoads = kKT * kChunks / 64;
  static constexpr int kPitch = D * 2 + 16;       // LDS bytes per V row (bank spread)
  static constexpr int kWaveLds = kKT * kPitch;
  static constexpr int kMergeRow = D + 4;         // floats per head row in the merge area
  static constexpr int kMergeBytes = (kWaves * 16 * kMergeRow + 2 * kWaves * 16) * 4;
  static constexpr int kLds = kWaves * kWaveLds > kMergeBytes ? kWaves * kWaveLds : kMergeBytes;
};

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int NHB>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(DecodeProblem p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::kLds];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
        if (key < j1) w = ld16(kb + int64_t(key) * D + (4 * ks + hi) * 8);
        kreg[blk][ks] = w;
      }
    }
#pragma unroll
    for (int t = 0; t < C::kVLoads; ++t) {
      const int idx = t * 64 + lane;
      const int key = jt + idx / C::kChunks;
      const int ch = idx % C::kChunks;
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (key < j1) w = ld16(vb + int64_t(key) * D + ch * 8);
      vreg[t] = w;
    }
  };

  int jt = j0 + wave * kKT;
  if (jt < j1) load_tile(jt);
  for (; jt < j1; jt += kWaves * kKT) {
    u32x4_t kc[2][C::kSteps];
    u32x4_t vc[C::kVLoads];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int ks = 0; ks < C::kSteps; ++ks) kc[blk][ks] = kreg[blk][ks];
#pragma unroll
    for (int t = 0; t < C::kVLoads; ++t) vc[t] = vreg[t];
    if (jt + kWaves * kKT < j1) load_tile(jt + kWaves * kKT);

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
      const float alpha = exp2f(mrun[hb] - mn);
      mrun[hb] = mn;
      uint32_t w[4];
      float lsum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          const uint32_t pk = pack_bf16x2(exp2f(t2[blk][2 * r2] - mn), exp2f(t2[blk][2 * r2 + 1] - mn));
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

  // merge the four waves, one head block at a time
  float* sm_o = reinterpret_cast<float*>(smem);
  float* sm_m = sm_o + kWaves * 16 * C::kMergeRow;
  float* sm_l = sm_m + kWaves * 16;
  constexpr int kC8 = D / 8;
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
    const int nh = min(16, p.n_rep - 16 * hb);
    for (int t = threadIdx.x; t < nh * kC8; t += 256) {
      const int hl = t / kC8;
      const int c8 = t % kC8;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (sm_l[w * 16 + hl] > 0.f) M = fmaxf(M, sm_m[w * 16 + hl]);
      float L = 0.f;
      float O[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float lw = sm_l[w * 16 + hl];
        if (lw > 0.f) {
          const float f = exp2f(sm_m[w * 16 + hl] - M);
          L = fmaf(lw, f, L);
          const float* src = sm_o + (w * 16 + hl) * C::kMergeRow + c8 * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) O[e] = fmaf(src[e], f, O[e]);
        }
      }
      const int h = g * p.n_rep + 16 * hb + hl;
      if (S == 1) {
        u32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(L > 0.f ? O[2 * e] / L : 0.f, L > 0.f ? O[2 * e + 1] / L : 0.f);
        st16(p.out + (int64_t(b) * p.H + h) * D + c8 * 8, w);
      } else {
        const int64_t pr = (int64_t(b) * p.H + h) * S + s;
        float* dst = p.part_o + pr * D + c8 * 8;
        st16(dst, u32x4_t{__float_as_uint(O[0]), __float_as_uint(O[1]), __float_as_uint(O[2]), __float_as_uint(O[3])});
        st16(dst + 4, u32x4_t{__float_as_uint(O[4]), __float_as_uint(O[5]), __float_as_uint(O[6]), __float_as_uint(O[7])});
        if (c8 == 0) {
          p.part_ml[pr * 2] = M;
          p.part_ml[pr * 2 + 1] = L;
        }
      }
    }
  }
}

template <int D, int NHB>
hipError_t launch_t(const DecodeProblem& p, hipStream_t stream) {
  const int64_t blocks = int64_t(p.B) * p.G * p.num_splits;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_mfma_kernel<D, NHB>), dim3(unsigned(blocks)), dim3(256), 0, stream, p);
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
