// Causal GQA prefill on the gfx950 matrix cores (bfloat16 in, float32 accumulate).
//
// Definition: query position i of head h attends keys 0..i of K/V head
// floor(h*G/H) through softmax(scale * q.k) and a weighted sum of v (fogdragon
// CSDN blog: the context phase runs in parallel over the prompt, each position
// seeing only its past; GQA paper section 2.2 for the grouping).
//
// Work unit: one workgroup of 4 waves per (b, g, head quad, query tile).  Each
// wave owns 32 query positions of one head; the 4 waves of a workgroup are the
// 4 heads of one group (n_rep >= 4) or 2/4 consecutive 32-position blocks of
// the group's heads (n_rep = 2/1), so every K/V tile staged in LDS is used by
// 128 query rows.  Per 64-key tile and wave:
//
//   S^T[key][row] = K[key][:] . Q[row][:]        32x32x16 bf16 MFMA (2 x 8),
//                   A = K tile from LDS (XOR-swizzled 16-byte chunks),
//                   B = the wave's queries (registers, loaded once)
//   mask j > i on tiles that reach the diagonal; online softmax in base 2,
//   float32, one query row per lane column (max/sum in-lane plus one exchange)
//   O^T[dim][row] += V^T[dim][key] P^T[key][row] 32x32x16 MFMA (4 x 4),
//                   A = V^T from LDS (transposed when staged),
//                   B = the weights, rounded to bf16, already in place
//
// Query tiles are issued heaviest (last) first so the causal triangle
// balances across the machine.

#include "device_common.h"
#include "internal.h"

namespace gqa {
namespace {

constexpr int kKT = 64;     // keys per tile
constexpr int kQT = 32;     // query positions per wave

template <int D>
struct PCfg {
  static constexpr int kSteps = D / 16;          // QK k-steps (k = 16)
  static constexpr int kColBlocks = D / 32;      // PV output blocks of 32 dims
  static constexpr int kChunks = D / 8;          // 16-byte chunks per row
  static constexpr int kLoads = kKT * kChunks / 256;   // per thread per tile (K and V each)
  static constexpr int kKBytes = kKT * D * 2;
  static constexpr int kVPitch = kKT * 2 + 16;   // bytes per V^T row
  static constexpr int kVBytes = D * kVPitch;
};

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of key kl (0..63) inside a V^T row: the 8 keys that one lane feeds
// to one PV k-step are contiguous.  kl = 16u + 8a + 4h + b  ->  16u + 8h + 4a + b.
__device__ __forceinline__ int vt_pos(int kl) {
  return (kl & ~15) | ((kl & 4) << 1) | ((kl & 8) >> 1) | (kl & 3);
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillProblem p) {
  using C = PCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::kKBytes + C::kVBytes];
  char* sk = smem;
  char* sv = smem + C::kKBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  const int nre = p.n_rep < 4 ? p.n_rep : 4;      // heads per workgroup
  const int tb_per_wg = 4 / nre;                   // 32-position blocks per workgroup
  const int n_hq = p.n_rep / nre;
  const int rows_wg = kQT * tb_per_wg;
  const int n_qt = (p.T + rows_wg - 1) / rows_wg;
  const int units = p.B * p.G * n_hq;
  const int qt = n_qt - 1 - int(blockIdx.x / unsigned(units));
  const int unit = int(blockIdx.x % unsigned(units));
  const int hq = unit % n_hq;
  const int g = (unit / n_hq) % p.G;
  const int b = unit / (n_hq * p.G);

  const int head = g * p.n_rep + hq * nre + (wave % nre);
  const int t_base = qt * rows_wg + (wave / nre) * kQT;
  const int t_row = t_base + l32;                  // this lane's query position
  const int t_last = min(p.T, (qt + 1) * rows_wg) - 1;
  const int n_kt = t_last / kKT + 1;

  // queries: B operand, lane column = row l32, k-slot group h2 -> dims 16*ks + 8*h2 .. +7
  bf16x8_t qop[C::kSteps];
  {
    const bool rv = t_row < p.T;
    const uint16_t* qrow = p.q + ((int64_t(b) * p.T + (rv ? t_row : 0)) * p.H + head) * D;
#pragma unroll
    for (int ks = 0; ks < C::kSteps; ++ks) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (rv) w = ld16(qrow + 16 * ks + 8 * h2);
      qop[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x16_t acc[C::kColBlocks];
#pragma unroll
  for (int cb = 0; cb < C::kColBlocks; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  float mrun = -INFINITY;
  float lrun = 0.f;
  const float c2 = p.scale * kLog2e;

  const int64_t kv_row = int64_t(p.G) * D;           // elements between positions
  const uint16_t* kbase = p.k + (int64_t(b) * p.T * p.G + g) * D;
  const uint16_t* vbase = p.v + (int64_t(b) * p.T * p.G + g) * D;

  u32x4_t kreg[C::kLoads], vreg[C::kLoads];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int item = i * 256 + tid;
      const int kl = item / C::kChunks;
      const int ch = item % C::kChunks;
      const int key = kt * kKT + kl;
      u32x4_t wk = {0u, 0u, 0u, 0u}, wv = {0u, 0u, 0u, 0u};
      if (key < p.T) {
        wk = ld16(kbase + int64_t(key) * kv_row + ch * 8);
        wv = ld16(vbase + int64_t(key) * kv_row + ch * 8);
      }
      kreg[i] = wk;
      vreg[i] = wv;
    }
  };

  load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();   // previous tile's LDS reads are done
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int item = i * 256 + tid;
      const int kl = item / C::kChunks;
      const int ch = item % C::kChunks;
      const int phys = ch ^ (kl & (C::kChunks - 1));
      *reinterpret_cast<u32x4_t*>(sk + kl * (D * 2) + phys * 16) = kreg[i];
      const int pos = vt_pos(kl);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = vreg[i][e];
        *reinterpret_cast<uint16_t*>(sv + (ch * 8 + 2 * e) * C::kVPitch + pos * 2) = uint16_t(w & 0xffffu);
        *reinterpret_cast<uint16_t*>(sv + (ch * 8 + 2 * e + 1) * C::kVPitch + pos * 2) = uint16_t(w >> 16);
      }
    }
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(kt + 1);

    const int key0 = kt * kKT;
    if (key0 > t_base + kQT - 1) continue;        // tile entirely after this wave's rows
    const bool diag = key0 + kKT - 1 > t_base;     // some key may follow some row

    // scores: lane holds S^T[key0 + 32*kb + 8*(r/4) + 4*h2 + r%4][t_row]
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t a;
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] = 0.f;
      const int kl = 32 * kb + l32;
#pragma unroll
      for (int ks = 0; ks < C::kSteps; ++ks) {
        const int phys = (2 * ks + h2) ^ (kl & (C::kChunks - 1));
        const u32x4_t kw = *reinterpret_cast<const u32x4_t*>(sk + kl * (D * 2) + phys * 16);
        a = mfma32(__builtin_bit_cast(bf16x8_t, kw), qop[ks], a);
      }
      sacc[kb] = a;
    }

    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[kb][r] * c2;
        if (diag) {
          const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
          x = (key > t_row || key >= p.T) ? -INFINITY : x;
        }
        sacc[kb][r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float mn = fmaxf(mrun, tmax);            // finite: key 0 precedes every row
    const float alpha = exp2f(mrun - mn);
    mrun = mn;

    // weights -> bf16 B operands, one per 16-key step u: keys 16u + 8*(e/4) + 4*h2 + e%4
    bf16x8_t pop[4];
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int r0 = 8 * (u & 1) + 2 * e2;
        const uint32_t pk = pack_bf16x2(exp2f(sacc[u >> 1][r0] - mn), exp2f(sacc[u >> 1][r0 + 1] - mn));
        w[e2] = pk;
        lsum += bf16lo_to_f32(pk) + bf16hi_to_f32(pk);
      }
      pop[u] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]});
    }
    lrun = fmaf(lrun, alpha, lsum);
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb) acc[cb] *= alpha;

#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int cb = 0; cb < C::kColBlocks; ++cb) {
        const int row = 32 * cb + l32;
        const u32x4_t vw = *reinterpret_cast<const u32x4_t*>(sv + row * C::kVPitch + (16 * u + 8 * h2) * 2);
        acc[cb] = mfma32(__builtin_bit_cast(bf16x8_t, vw), pop[u], acc[cb]);
      }
    }
  }

  const float l = lrun + shfl_xor(lrun, 32);
  if (t_row < p.T) {
    const float inv = 1.f / l;
    uint16_t* orow = p.out + ((int64_t(b) * p.T + t_row) * p.H + head) * D;
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = 32 * cb + 8 * r4 + 4 * h2;
        const uint32_t w0 = pack_bf16x2(acc[cb][4 * r4] * inv, acc[cb][4 * r4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(acc[cb][4 * r4 + 2] * inv, acc[cb][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + col) = make_uint2(w0, w1);
      }
  }
}

}  // namespace

bool prefill_mfma_supports(int n_rep, int d) {
  return (d == 64 || d == 128) && (n_rep == 1 || n_rep == 2 || n_rep % 4 == 0);
}

hipError_t launch_prefill_mfma(const PrefillProblem& p, hipStream_t stream) {
  const int nre = p.n_rep < 4 ? p.n_rep : 4;
  const int rows_wg = kQT * (4 / nre);
  const int64_t n_qt = (p.T + rows_wg - 1) / rows_wg;
  const int64_t blocks = n_qt * p.B * p.G * (p.n_rep / nre);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.d == 128)
    hipLaunchKernelGGL(prefill_mfma_kernel<128>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_mfma_kernel<64>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
