// kv_meanpool_heads: MHA -> GQA conversion of one K or V projection.
//
// GQA paper section 2.1 (Figure 1) and section 2.2; 2kiu.com tutorial section
// 4.3, step 2: each group's key (or value) projection is the mean of its member
// heads' projections.  Groups are consecutive blocks of n_rep heads.
//
// HBM-bound: every input element is read once and every output element
// written once.  Each thread owns 8 consecutive elements of one group's output
// (16-byte bfloat16 or 2 x 16-byte float32 accesses), reads the same 8 elements
// of the group's n_rep heads (up to 8 loads in flight, non-temporal: each input
// element is read once), sums in float32 in head order, divides once
// (correctly rounded) and rounds once to the storage type.  A grid-stride loop
// covers the output; a scalar kernel handles sizes that are not a multiple of 8.
// Several projections of one shape can go in one launch (grid row y =
// projection y): the launch's fixed cost is then paid once for all of them.

#include "device_common.h"
#include "internal.h"

namespace gqa {
namespace {

// Adds heads k0 .. k0+NB-1 of group g (8 elements at e8) to acc: all NB loads
// are issued before the first add, so NB requests per thread are in flight;
// the adds run in head order (the same rounding as one head at a time).
template <int DT, int NB>
__device__ __forceinline__ void add_heads(const MeanpoolProblem& p, const void* w_in, int64_t g, int64_t e8, int k0,
                                          float* acc) {
  if constexpr (DT != kF32) {
    u32x4_t w[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      w[j] = ld16_stream(static_cast<const uint16_t*>(w_in) + (g * p.n_rep + k0 + j) * p.per_head_elems + e8 * 8);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[2 * t] += Half16<DT>::lo(w[j][t]);
        acc[2 * t + 1] += Half16<DT>::hi(w[j][t]);
      }
  } else {
    u32x4_t a[NB], b[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float* src = static_cast<const float*>(w_in) + (g * p.n_rep + k0 + j) * p.per_head_elems + e8 * 8;
      a[j] = ld16_stream(src);
      b[j] = ld16_stream(src + 4);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[t] += __uint_as_float(a[j][t]);
        acc[4 + t] += __uint_as_float(b[j][t]);
      }
  }
}

template <int DT>
__global__ __launch_bounds__(256) void meanpool_vec8_kernel(MeanpoolProblem p) {
  const void* w_in = p.w_in[blockIdx.y];
  void* w_out = p.w_out[blockIdx.y];
  const int64_t vec_per_head = p.per_head_elems / 8;
  const int64_t total = int64_t(p.G) * vec_per_head;
  const float n = float(p.n_rep);
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t g = i / vec_per_head;
    const int64_t e8 = i - g * vec_per_head;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int k = 0;
    for (; k + 8 <= p.n_rep; k += 8) add_heads<DT, 8>(p, w_in, g, e8, k, acc);
    if (k + 4 <= p.n_rep) {
      add_heads<DT, 4>(p, w_in, g, e8, k, acc);
      k += 4;
    }
    for (; k < p.n_rep; ++k) add_heads<DT, 1>(p, w_in, g, e8, k, acc);
    const int64_t oel = g * p.per_head_elems + e8 * 8;
    if constexpr (DT != kF32) {
      u32x4_t w;
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = Half16<DT>::pack2(acc[2 * t] / n, acc[2 * t + 1] / n);
      st16(static_cast<uint16_t*>(w_out) + oel, w);
    } else {
      u32x4_t a, b;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = __float_as_uint(acc[t] / n);
        b[t] = __float_as_uint(acc[4 + t] / n);
      }
      float* dst = static_cast<float*>(w_out) + oel;
      st16(dst, a);
      st16(dst + 4, b);
    }
  }
}

template <int DT>
__global__ __launch_bounds__(256) void meanpool_scalar_kernel(MeanpoolProblem p) {
  const void* w_in = p.w_in[blockIdx.y];
  void* w_out = p.w_out[blockIdx.y];
  const int64_t total = int64_t(p.G) * p.per_head_elems;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t g = i / p.per_head_elems;
    const int64_t e = i - g * p.per_head_elems;
    float acc = 0.f;
    for (int k = 0; k < p.n_rep; ++k) {
      const int64_t elem = (g * p.n_rep + k) * p.per_head_elems + e;
      if constexpr (DT == kF32)
        acc += static_cast<const float*>(w_in)[elem];
      else
        acc += Half16<DT>::lo(static_cast<const uint16_t*>(w_in)[elem]);
    }
    const float mean = acc / float(p.n_rep);
    if constexpr (DT == kF32)
      static_cast<float*>(w_out)[i] = mean;
    else
      static_cast<uint16_t*>(w_out)[i] = uint16_t(Half16<DT>::pack2(mean, 0.f) & 0xffffu);
  }
}

}  // namespace

hipError_t launch_meanpool(const MeanpoolProblem& p, hipStream_t stream) {
  if (!abi_ok(p)) return kAbiMismatch;
  const bool vec = (p.per_head_elems % 8) == 0;
  const int64_t work = vec ? int64_t(p.G) * (p.per_head_elems / 8) : int64_t(p.G) * p.per_head_elems;
  if (p.count < 1 || p.count > kMaxMeanpoolBatch) return hipErrorInvalidValue;
  // enough threads to cover each projection's output once, capped (grid-stride
  // beyond); grid row y is projection y
  int64_t blocks = (work + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (blocks < 1) blocks = 1;
  const dim3 grid = dim3(unsigned(blocks), unsigned(p.count)), block = dim3(256);
  if (vec) {
    if (p.dtype == kBF16)
      hipLaunchKernelGGL(meanpool_vec8_kernel<kBF16>, grid, block, 0, stream, p);
    else if (p.dtype == kF16)
      hipLaunchKernelGGL(meanpool_vec8_kernel<kF16>, grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL(meanpool_vec8_kernel<kF32>, grid, block, 0, stream, p);
  } else {
    if (p.dtype == kBF16)
      hipLaunchKernelGGL(meanpool_scalar_kernel<kBF16>, grid, block, 0, stream, p);
    else if (p.dtype == kF16)
      hipLaunchKernelGGL(meanpool_scalar_kernel<kF16>, grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL(meanpool_scalar_kernel<kF32>, grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace gqa
