// Merge of split-N partial results (second pass of a split decode).
//
// Each split s of a (row, head) left its running maximum m_s (base-2 units),
// normaliser l_s and unnormalised output o_s.  The exact softmax over the
// union of the splits is
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s,
// taken over the splits that saw at least one position (l_s > 0); a row whose
// splits are all empty gets zeros.  One wave per (row, head), lanes across d.

#include "device_common.h"
#include "internal.h"

namespace gqa {
namespace {

template <int DT>
__global__ __launch_bounds__(256) void combine_kernel(CombineProblem p) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= int64_t(p.n_rows) * p.H) return;
  const int S = p.num_splits;
  const float* ml = p.part_ml + pair * S * 2;
  const float* po = p.part_o + pair * S * p.d;

  float M = -INFINITY;
  for (int s = 0; s < S; ++s)
    if (ml[2 * s + 1] > 0.f) M = fmaxf(M, ml[2 * s]);

  for (int col = lane; col < p.d; col += 64) {
    float L = 0.f, O = 0.f;
    for (int s = 0; s < S; ++s) {
      const float ls = ml[2 * s + 1];
      if (ls > 0.f) {
        const float f = exp2f(ml[2 * s] - M);
        L = fmaf(ls, f, L);
        O = fmaf(po[int64_t(s) * p.d + col], f, O);
      }
    }
    const float val = L > 0.f ? O / L : 0.f;
    const int64_t row = pair / p.H;
    const int h = int(pair - row * p.H);
    const int64_t oi = (row * p.hm.o_heads + p.hm.o_head(h / p.n_rep, h % p.n_rep)) * p.d + col;
    if (DT == kF32)
      static_cast<float*>(p.out)[oi] = val;
    else if (DT == kF16)
      static_cast<uint16_t*>(p.out)[oi] = to_f16(val);
    else
      static_cast<uint16_t*>(p.out)[oi] = to_bf16(val);
  }
}

}  // namespace

hipError_t launch_combine(const CombineProblem& p, hipStream_t stream) {
  if (!abi_ok(p)) return kAbiMismatch;
  const int64_t pairs = int64_t(p.n_rows) * p.H;
  const int64_t blocks = (pairs + 3) / 4;
  if (blocks <= 0) return hipSuccess;
  if (p.dtype == kF32)
    hipLaunchKernelGGL(combine_kernel<kF32>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  else if (p.dtype == kF16)
    hipLaunchKernelGGL(combine_kernel<kF16>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<kBF16>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
