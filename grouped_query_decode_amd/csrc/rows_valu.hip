// Vector-unit attention of query rows over a K/V head, for any (n_rep, dtype).
//
// Serves float32 decode, float32 causal prefill, and bfloat16 shapes the
// matrix-core kernels do not cover.  Definition (fogdragon CSDN blog, section
// "KV Cache"; GQA paper section 2.2): for query row z and head h of group g,
//   out = sum_j softmax_j(scale * q . K[j]) V[j]   over the attended positions.
//
// Work unit: one workgroup (4 waves) per (row, K/V head, split, block of up to
// 8 heads of the group; the block size is a template parameter, the smallest
// of 1, 2, 4, 8 that holds the group).  Each cached position is read once per
// unit and used by all heads of the block.  A position's d elements are spread
// over a lane group of d*sizeof/16 lanes (one 16-byte load each); several
// lane groups, each with positions of its own, share a wave instruction.
// Softmax is online, in base 2, in float32, and every lane group keeps its own
// running (max, sum, output): inside the loop the only cross-lane step is the
// dot product's sum over the lane group, and the heads' chains are independent
// (no early exit), so their latencies overlap.  The lane groups, then the four
// waves, merge their (max, sum, output) at the end.

#include "device_common.h"
#include "internal.h"

namespace gqa {
namespace {

constexpr int kMaxHeadsPerBlock = 8;
constexpr int kWaves = 4;

template <int DT>
struct Elem;
template <>
struct Elem<kF32> {
  static constexpr int kSize = 4;
  __device__ static void load16(const char* p, float* f) {
    u32x4_t w = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
  __device__ static void store(char* p, int i, float x) { reinterpret_cast<float*>(p)[i] = x; }
};
template <>
struct Elem<kBF16> {
  static constexpr int kSize = 2;
  __device__ static void load16(const char* p, float* f) {
    u32x4_t w = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16lo_to_f32(w[i]);
      f[2 * i + 1] = bf16hi_to_f32(w[i]);
    }
  }
  __device__ static void store(char* p, int i, float x) {
    reinterpret_cast<uint16_t*>(p)[i] = to_bf16(x);
  }
};

template <>
struct Elem<kF16> {
  static constexpr int kSize = 2;
  __device__ static void load16(const char* p, float* f) {
    u32x4_t w = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16lo_to_f32(w[i]);
      f[2 * i + 1] = f16hi_to_f32(w[i]);
    }
  }
  __device__ static void store(char* p, int i, float x) {
    reinterpret_cast<uint16_t*>(p)[i] = to_f16(x);
  }
};

template <int DT, int D, int kHeadsPerBlock>
__global__ __launch_bounds__(256) void rows_valu_kernel(RowsProblem p) {
  using E = Elem<DT>;
  constexpr int EPL = 16 / E::kSize;   // elements per lane
  constexpr int LPR = D / EPL;         // lanes per cached position
  constexpr int RPW = 64 / LPR;        // positions per wave step
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "layout");

  __shared__ float sm_m[kWaves][kHeadsPerBlock];
  __shared__ float sm_l[kWaves][kHeadsPerBlock];
  __shared__ float sm_o[kWaves][kHeadsPerBlock][D];
  static_assert(kHeadsPerBlock >= 1 && kHeadsPerBlock <= kMaxHeadsPerBlock, "head block");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;
  const int c = lane % LPR;

  const int n_hb = (p.n_rep + kHeadsPerBlock - 1) / kHeadsPerBlock;
  int64_t bid = blockIdx.x;
  const int hb = int(bid % n_hb);
  bid /= n_hb;
  const int s = int(bid % p.num_splits);
  bid /= p.num_splits;
  const int g = int(bid % p.G);
  const int z = int(bid / p.G);
  const int b = z / p.rows_per_batch;

  int len;
  if (p.causal) {
    const int ctx = p.ctx_lens ? max(p.ctx_lens[b], 0) : 0;
    len = min(ctx + z % p.rows_per_batch + 1, p.n_max);
  } else {
    len = p.seqlens[b];
    len = len < 0 ? 0 : (len > p.n_max ? p.n_max : len);
  }
  const int j0 = s * p.split_len;
  const int j1 = min(len, j0 + p.split_len);
  const int r0 = hb * kHeadsPerBlock;             // first query of the group in this block
  const int h0 = g * p.n_rep + r0;
  const int nh = min(kHeadsPerBlock, p.n_rep - r0);

  // Query chunk of every head, pre-multiplied by scale*log2(e) so that the
  // scores come out in base-2 units.
  const float qmul = p.scale * kLog2e;
  float qf[kHeadsPerBlock][EPL];
  const char* qrow = static_cast<const char*>(p.q) + (int64_t(z) * p.hm.q_heads * D) * E::kSize;
#pragma unroll
  for (int hh = 0; hh < kHeadsPerBlock; ++hh) {
    if (hh < nh) {
      E::load16(qrow + (p.hm.q_head(g, r0 + hh) * D + c * EPL) * E::kSize, qf[hh]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[hh][e] *= qmul;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[hh][e] = 0.f;
    }
  }

  float m[kHeadsPerBlock], l[kHeadsPerBlock], o[kHeadsPerBlock][EPL];
#pragma unroll
  for (int hh = 0; hh < kHeadsPerBlock; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[hh][e] = 0.f;
  }

  const int64_t kv_off = int64_t(b) * p.kv_batch_stride + int64_t(g) * p.kv_group_stride;
  const char* kbase = static_cast<const char*>(p.k) + kv_off * E::kSize;
  const char* vbase = static_cast<const char*>(p.v) + kv_off * E::kSize;

  // Positions in batches of kUnroll wave steps: all their loads are issued
  // before any of them is used, so the load latency is paid once per batch.
  // A one-head block has the registers for eight steps (the 128-position
  // float32 decode then waits for one batch instead of two: 4.7 us, not 5.0).
  constexpr int kUnroll = kHeadsPerBlock == 1 ? 8 : 4;
  for (int jb = j0 + wave * RPW; jb < j1; jb += kWaves * RPW * kUnroll) {
    float kf[kUnroll][EPL], vf[kUnroll][EPL];
    bool valid[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = jb + u * kWaves * RPW + r;
      valid[u] = j < j1;
      if (valid[u]) {
        const int64_t off = (int64_t(j) * p.kv_pos_stride + c * EPL) * E::kSize;
        E::load16(kbase + off, kf[u]);
        E::load16(vbase + off, vf[u]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kf[u][e] = vf[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int hh = 0; hh < kHeadsPerBlock; ++hh) {
        float sc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) sc = fmaf(qf[hh][e], kf[u][e], sc);
        sc = lane_group_sum<LPR>(sc);
        sc = valid[u] ? sc : -INFINITY;
        // this lane group's running maximum (-inf until its first valid position)
        const float mn = fmaxf(m[hh], sc);
        const float alpha = mn == -INFINITY ? 1.f : exp2f(m[hh] - mn);
        const float pj = valid[u] ? exp2f(sc - mn) : 0.f;
        l[hh] = fmaf(l[hh], alpha, pj);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[hh][e] = fmaf(pj, vf[u][e], o[hh][e] * alpha);
        m[hh] = mn;
      }
    }
  }

  // Merge the lane groups of the wave: rescale each to the wave's maximum,
  // then sum (max, sum, output) over the groups.
#pragma unroll
  for (int hh = 0; hh < kHeadsPerBlock; ++hh) {
    float mw = m[hh];
#pragma unroll
    for (int msk = LPR; msk < 64; msk <<= 1) mw = fmaxf(mw, shfl_xor(mw, msk));
    const float f = mw == -INFINITY ? 0.f : exp2f(m[hh] - mw);
    float lw = l[hh] * f;
#pragma unroll
    for (int msk = LPR; msk < 64; msk <<= 1) lw += shfl_xor(lw, msk);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = o[hh][e] * f;
#pragma unroll
      for (int msk = LPR; msk < 64; msk <<= 1) x += shfl_xor(x, msk);
      o[hh][e] = x;
    }
    m[hh] = mw;
    l[hh] = lw;
  }
  if (lane < LPR) {
#pragma unroll
    for (int hh = 0; hh < kHeadsPerBlock; ++hh)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][hh][c * EPL + e] = o[hh][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < kHeadsPerBlock; ++hh) {
      sm_m[wave][hh] = m[hh];
      sm_l[wave][hh] = l[hh];
    }
  }
  __syncthreads();

  for (int t = threadIdx.x; t < nh * D; t += blockDim.x) {
    const int hh = t / D;
    const int col = t % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (sm_l[w][hh] > 0.f) M = fmaxf(M, sm_m[w][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (sm_l[w][hh] > 0.f) {
        const float f = exp2f(sm_m[w][hh] - M);
        L = fmaf(sm_l[w][hh], f, L);
        O = fmaf(sm_o[w][hh][col], f, O);
      }
    }
    const int h = h0 + hh;
    if (p.num_splits == 1) {
      char* orow = static_cast<char*>(p.out) +
                   ((int64_t(z) * p.hm.o_heads + p.hm.o_head(g, r0 + hh)) * D) * E::kSize;
      E::store(orow, col, L > 0.f ? O / L : 0.f);
    } else {
      const int64_t pr = (int64_t(z) * p.H + h) * p.num_splits + s;
      p.part_o[pr * D + col] = O;
      if (col == 0) {
        p.part_ml[pr * 2] = M;
        p.part_ml[pr * 2 + 1] = L;
      }
    }
  }
}

template <int DT, int D, int HB>
hipError_t launch_hb(const RowsProblem& p, hipStream_t stream) {
  const int n_hb = (p.n_rep + HB - 1) / HB;
  const int64_t blocks = int64_t(p.n_rows) * p.G * p.num_splits * n_hb;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((rows_valu_kernel<DT, D, HB>), dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// The smallest head block that holds the group (no padded heads below 8) --
// halved while that leaves fewer workgroups than compute units: a small
// problem then runs one or two heads per workgroup, many workgroups reading
// the same rows (the repeats come from the caches), so that each workgroup's
// dependent chain of softmax steps is short.
template <int DT, int D>
hipError_t launch_t(const RowsProblem& p, hipStream_t stream) {
  int hb = p.n_rep <= 1 ? 1 : (p.n_rep <= 2 ? 2 : (p.n_rep <= 4 ? 4 : 8));
  const int64_t units = int64_t(p.n_rows) * p.G * p.num_splits;
  while (hb > 1 && units * ((p.n_rep + hb - 1) / hb) < 256) hb /= 2;
  switch (hb) {
    case 1: return launch_hb<DT, D, 1>(p, stream);
    case 2: return launch_hb<DT, D, 2>(p, stream);
    case 4: return launch_hb<DT, D, 4>(p, stream);
    default: return launch_hb<DT, D, 8>(p, stream);
  }
}

}  // namespace

hipError_t launch_rows_valu(const RowsProblem& p, int dtype, hipStream_t stream) {
  if (!abi_ok(p)) return kAbiMismatch;
  if (dtype == kF32) {
    return p.d == 64 ? launch_t<kF32, 64>(p, stream) : launch_t<kF32, 128>(p, stream);
  }
  if (dtype == kF16) {
    return p.d == 64 ? launch_t<kF16, 64>(p, stream) : launch_t<kF16, 128>(p, stream);
  }
  return p.d == 64 ? launch_t<kBF16, 64>(p, stream) : launch_t<kBF16, 128>(p, stream);
}

}  // namespace gqa
