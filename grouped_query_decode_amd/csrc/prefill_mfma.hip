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
//                   A = K tile from LDS, B = the wave's queries (registers)
//   mask j > i on tiles that reach the diagonal; online softmax in base 2,
//   float32, one query row per lane column (max/sum in-lane plus one exchange)
//   O^T[dim][row] += V^T[dim][key] P^T[key][row] 32x32x16 MFMA (4 x 4),
//                   A = V^T read from the row-major V tile with the gfx950
//                   transposing LDS load, B = the bf16 weights, already in place
//
// K/V tiles are double-buffered in LDS (row-major, rows padded so that the
// operand reads hit distinct banks): the next tile's
// global loads are issued before the current tile's math and land in the other
// buffer afterwards, one barrier per tile.  Softmax work per score: one FMA
// (scale folded in), one hardware exp2 (weights below 2^-126 may flush to
// zero), a third of a max3, half a bf16 pack, half a
// bf16 dot2 for the normaliser (which sums the rounded weights); the running
// output is rescaled only when some row's maximum grew.  Query tiles are issued
// heaviest first, and the query tiles of a (b, g) stay on one XCD (consecutive
// workgroups go to consecutive XCDs) so its K/V stays in that XCD's L2.

#include "device_common.h"
#include "internal.h"

namespace gqa {
namespace {

constexpr int kKT = 64;     // keys per tile
constexpr int kQT = 32;     // query positions per wave
constexpr int kXcds = 8;

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// LDS tile rows are padded so that the operand reads hit distinct banks
// (64 banks of 4 bytes): a K row is 16 bytes longer than its data (16
// consecutive rows read at one column cover all banks with 16-byte reads), a
// V row 32 bytes longer (the transposing reads of 4 rows x 2 chunks by a
// 16-lane group cover 32 distinct banks).  Every operand address is then a
// per-lane base plus a compile-time offset.
template <int D>
struct PCfg {
  static constexpr int kSteps = D / 16;          // QK k-steps (k = 16)
  static constexpr int kColBlocks = D / 32;      // PV output blocks of 32 dims
  static constexpr int kChunks = D / 8;          // 16-byte chunks per row
  static constexpr int kLoads = kKT * kChunks / 256;   // per thread per tile (K and V each)
  static constexpr int kKPitch = D * 2 + 16;
  static constexpr int kVPitch = D * 2 + 32;
  static constexpr int kKBytes = kKT * kKPitch;
  static constexpr int kVBytes = kKT * kVPitch;
  static constexpr int kBufBytes = kKBytes + kVBytes;
};

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// gfx950 transposing LDS read: within each 16-lane group, lanes 4e..4e+3
// address row e (4 consecutive bf16 each) of a 4 x 16 block, and lane i
// receives column i of the 4 rows.
__device__ __forceinline__ i16x4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(const_cast<char*>(p)));
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillProblem p) {
  using C = PCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kBufBytes];   // K0 V0 K1 V1

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
  int unit, qt_rank;
  if (units % kXcds == 0) {
    // keep a unit's query tiles on one XCD: workgroup i runs on XCD i % 8
    const int x = int(blockIdx.x % kXcds);
    const int i = int(blockIdx.x / kXcds);
    const int per_xcd = units / kXcds;
    unit = x * per_xcd + i % per_xcd;
    qt_rank = i / per_xcd;
  } else {
    unit = int(blockIdx.x % unsigned(units));
    qt_rank = int(blockIdx.x / unsigned(units));
  }
  const int qt = n_qt - 1 - qt_rank;              // heaviest first
  const int hq = unit % n_hq;
  const int g = (unit / n_hq) % p.G;
  const int b = unit / (n_hq * p.G);

  const int head = g * p.n_rep + hq * nre + (wave % nre);
  const int t_base = qt * rows_wg + (wave / nre) * kQT;
  const int t_row = t_base + l32;                  // this lane's query position
  const int t_last = min(p.T, (qt + 1) * rows_wg) - 1;
  const int n_kt = t_last / kKT + 1;

  // queries: B operand, lane column = row l32, k-slot group h2 -> dims 16*ks + 8*h2 .. +7.
  // A negative scale is folded into the queries (exact sign flip).
  const uint32_t qsign = p.scale < 0.f ? 0x80008000u : 0u;
  // (a zero scale is replaced by a tiny one: the weights are then exactly
  // uniform, and masked scores still map to exactly zero weight)
  const float c2 = p.scale == 0.f ? 1e-30f : fabsf(p.scale) * kLog2e;
  bf16x8_t qop[C::kSteps];
  {
    const bool rv = t_row < p.T;
    const uint16_t* qrow = p.q + ((int64_t(b) * p.T + (rv ? t_row : 0)) * p.H + head) * D;
#pragma unroll
    for (int ks = 0; ks < C::kSteps; ++ks) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (rv) w = ld16(qrow + 16 * ks + 8 * h2);
      w ^= u32x4_t{qsign, qsign, qsign, qsign};
      qop[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x16_t acc[C::kColBlocks];
#pragma unroll
  for (int cb = 0; cb < C::kColBlocks; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  float mrun = -INFINITY;     // running max of the raw scores of this lane's row
  float lrun = 0.f;           // this lane's share of the normaliser

  const int64_t kv_row = int64_t(p.G) * D;           // elements between positions
  const uint16_t* kbase = p.k + (int64_t(b) * p.T * p.G + g) * D;
  const uint16_t* vbase = p.v + (int64_t(b) * p.T * p.G + g) * D;

  u32x4_t kreg[C::kLoads], vreg[C::kLoads];
  // thread's first (position, chunk) of a tile; the others are 256/kChunks positions apart
  const int kl0 = tid / C::kChunks;
  const int ch0 = tid % C::kChunks;
  constexpr int kRowStep = 256 / C::kChunks;
  auto load_tile = [&](int kt) {
    const int key0 = kt * kKT + kl0;
    const uint16_t* kp = kbase + int64_t(key0) * kv_row + ch0 * 8;
    const uint16_t* vp = vbase + int64_t(key0) * kv_row + ch0 * 8;
    if (kt * kKT + kKT <= p.T) {                   // whole tile inside the prompt
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i) {
        kreg[i] = ld16(kp + int64_t(i * kRowStep) * kv_row);
        vreg[i] = ld16(vp + int64_t(i * kRowStep) * kv_row);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i) {
        u32x4_t wk = {0u, 0u, 0u, 0u}, wv = {0u, 0u, 0u, 0u};
        if (key0 + i * kRowStep < p.T) {
          wk = ld16(kp + int64_t(i * kRowStep) * kv_row);
          wv = ld16(vp + int64_t(i * kRowStep) * kv_row);
        }
        kreg[i] = wk;
        vreg[i] = wv;
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* sk = smem + buf * C::kBufBytes;
    char* sv = sk + C::kKBytes;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      *reinterpret_cast<u32x4_t*>(sk + (kl0 + i * kRowStep) * C::kKPitch + ch0 * 16) = kreg[i];
      *reinterpret_cast<u32x4_t*>(sv + (kl0 + i * kRowStep) * C::kVPitch + ch0 * 16) = vreg[i];
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);
    const char* sk = smem + buf * C::kBufBytes;
    const char* sv = sk + C::kKBytes;

    const int key0 = kt * kKT;
    if (key0 <= t_base + kQT - 1) {                 // some key precedes some row of this wave
      const bool diag = key0 + kKT - 1 > t_base;    // some key may follow some row

      // scores: lane holds S^T[key0 + 32*kb + 8*(r/4) + 4*h2 + r%4][t_row]
      f32x16_t sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16_t a;
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = 0.f;
        const char* krow = sk + (32 * kb + l32) * C::kKPitch + h2 * 16;
#pragma unroll
        for (int ks = 0; ks < C::kSteps; ++ks) {
          const u32x4_t kw = *reinterpret_cast<const u32x4_t*>(krow + ks * 32);
          a = mfma32(__builtin_bit_cast(bf16x8_t, kw), qop[ks], a);
        }
        sacc[kb] = a;
      }

      if (diag) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
            if (key > t_row || key >= p.T) sacc[kb][r] = -INFINITY;
          }
      }
      float tmax = mrun;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) tmax = fmaxf(fmaxf(tmax, sacc[kb][r]), sacc[kb][r + 1]);
      const float mn = fmaxf(tmax, shfl_xor(tmax, 32));   // finite: key 0 precedes every row
      const float mc = mn * c2;
      if (__any(mn != mrun)) {                     // some row's maximum grew: rescale
        const float alpha = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun * c2 - mc);
        lrun *= alpha;
#pragma unroll
        for (int cb = 0; cb < C::kColBlocks; ++cb) acc[cb] *= alpha;
        mrun = mn;
      }

      // weights -> bf16 B operands, one per 16-key step u: keys 16u + 8*(e/4) + 4*h2 + e%4
      bf16x8_t pop[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int r0 = 8 * (u & 1) + 2 * e2;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[u >> 1][r0], c2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[u >> 1][r0 + 1], c2, -mc));
          w[e2] = pack_bf16x2(p0, p1);
          lrun = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e2]),
                                                 __builtin_bit_cast(bf16x2_t, 0x3f803f80u), lrun, false);
        }
        pop[u] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]});
      }

      // O^T += V^T P^T; V^T operand via transposing reads of the row-major V tile:
      // lane (16-lane group grp, index i) gets column 32*cb + 16*(grp%2) + i of
      // keys 16u + 4*h2 + 0..3 (first read) and 16u + 8 + 4*h2 + 0..3 (second).
      const int grp = lane >> 4;
      const int li = lane & 15;
      // lane's address inside the 4 x 16 block it helps read: row li/4, columns 4*(li%4)..+3
      const char* vlane = sv + (4 * h2 + (li >> 2)) * C::kVPitch + (16 * (grp & 1) + 4 * (li & 3)) * 2;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int cb = 0; cb < C::kColBlocks; ++cb) {
          const char* a0 = vlane + (16 * u) * C::kVPitch + 64 * cb;
          const i16x4_t lo4 = lds_read_tr16(a0);
          const i16x4_t hi4 = lds_read_tr16(a0 + 8 * C::kVPitch);
          const bf16x8_t vop = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[cb] = mfma32(vop, pop[u], acc[cb]);
        }
      }
    }

    if (kt + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
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
