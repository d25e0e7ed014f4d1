// KV-cache append: this step's k and v rows go to cache position seqlens[b]-1.
//
// Definition: fogdragon CSDN blog, section "KV Cache" -- each step concatenates
// its new k and v onto the cached K and V before attending.  With a cache of
// n_max slots and a length that already counts the new token, that is slot
// seqlens[b]-1; a length of 0 (no token) or above n_max (no such slot) writes
// nothing.  The bf16 decode kernel does this inside its own launch; this
// kernel serves the float32 path, which runs it just before the decode.

#include "device_common.h"
#include "internal.h"

namespace gqa {
namespace {

__global__ __launch_bounds__(64) void append_kernel(AppendProblem p) {
  const int chunks = p.row_bytes / 16;
  for (int64_t unit = blockIdx.x; unit < int64_t(p.B) * p.G; unit += gridDim.x) {
    const int b = int(unit / p.G);
    const int len = p.seqlens[b];
    if (len < 1 || len > p.n_max) continue;
    const int64_t src = unit * p.row_bytes;
    const int64_t dst = (unit * p.n_max + (len - 1)) * p.row_bytes;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
      st16(static_cast<char*>(p.k) + dst + c * 16, ld16(static_cast<const char*>(p.k_new) + src + c * 16));
      st16(static_cast<char*>(p.v) + dst + c * 16, ld16(static_cast<const char*>(p.v_new) + src + c * 16));
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendProblem& p, hipStream_t stream) {
  if (!abi_ok(p)) return kAbiMismatch;
  const int64_t units = int64_t(p.B) * p.G;
  if (units <= 0) return hipSuccess;
  const unsigned blocks = unsigned(units < 65536 ? units : 65536);
  hipLaunchKernelGGL(append_kernel, dim3(blocks), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
