// Achievable HBM read bandwidth on gfx950, for the benchmark's ceiling: every
// lane streams 16-byte loads with the non-temporal hint (the data is read
// once and should not displace cached lines), U loads in flight per lane per
// iteration, over a buffer much larger than the 256 MB last-level cache.  The
// loaded words are folded into one value that is stored only if it equals an
// impossible key, so no load can be optimised away and almost nothing is
// written.  This is measurement code, separate from libgqa.so.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/gqa_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int U>
__global__ __launch_bounds__(kThreads) void hbm_read_probe_kernel(const u32x4_t* __restrict__ p, int64_t n16,
                                                                  uint32_t* sink, uint32_t key) {
  u32x4_t acc = {0u, 0u, 0u, 0u};
  const int64_t stride = int64_t(gridDim.x) * kThreads * U;
  int64_t i = int64_t(blockIdx.x) * kThreads * U + threadIdx.x;
  // whole chunks: this lane's U elements i, i + 256, ..., i + 256 (U - 1) are all below n16
  for (; i + int64_t(U - 1) * kThreads < n16; i += stride) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  // the one partial chunk left, element by element
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (i + int64_t(u) * kThreads < n16) acc ^= __builtin_nontemporal_load(p + i + u * kThreads);
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == key) sink[0] = 1u;
}

template <int U>
hipError_t launch(const void* buf, int64_t n16, uint32_t* sink, int blocks, hipStream_t s) {
  hipLaunchKernelGGL((hbm_read_probe_kernel<U>), dim3(unsigned(blocks)), dim3(kThreads), 0, s,
                     static_cast<const u32x4_t*>(buf), n16, sink, 0x9e3779b9u);
  return hipGetLastError();
}

}  // namespace

extern "C" int gqa_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, int unroll,
                                  void* stream) {
  if (!buf || !sink || bytes == 0 || (bytes & 15u) || (reinterpret_cast<uintptr_t>(buf) & 15u) ||
      (reinterpret_cast<uintptr_t>(sink) & 3u) || blocks < 1 || blocks > (1 << 20))
    return 1;
  const int64_t n16 = int64_t(bytes / 16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (unroll) {
    case 4: e = launch<4>(buf, n16, sink, blocks, s); break;
    case 8: e = launch<8>(buf, n16, sink, blocks, s); break;
    case 16: e = launch<16>(buf, n16, sink, blocks, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 4;
}

// ---------------------------------------------------------------------------
// Vector-unit issue rates: every lane runs 8 independent chains of N steps of
// one instruction kind (kind 0: v_fma_f32; 1: v_exp_f32; 2: one of each per
// step), so the time of a launch over the whole chip gives the SIMD cycles per
// wave64 instruction of that kind (and whether an exp overlaps an FMA).
// ---------------------------------------------------------------------------
namespace {

constexpr int kRateSteps = 4096;

template <int KIND>
__global__ __launch_bounds__(kThreads) void valu_rate_kernel(float* out, float seed) {
  float x[8], y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = seed * float(threadIdx.x + j);
    y[j] = seed * float(j);
  }
  for (int i = 0; i < kRateSteps; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (KIND != 0) x[j] = __builtin_amdgcn_exp2f(-fabsf(x[j]));
      if constexpr (KIND != 1) y[j] = fmaf(y[j], 0.999f, 0.0001f);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) r += x[j] + y[j];
  out[int64_t(blockIdx.x) * kThreads + threadIdx.x] = r;
}

}  // namespace

extern "C" int gqa_probe_valu_rate(float* out, int kind, int blocks, void* stream) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 3u) || blocks < 1 || blocks > (1 << 16) || kind < 0 || kind > 2)
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(valu_rate_kernel<0>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, out, 0.001f);
  else if (kind == 1)
    hipLaunchKernelGGL(valu_rate_kernel<1>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, out, 0.001f);
  else
    hipLaunchKernelGGL(valu_rate_kernel<2>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, out, 0.001f);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// ---------------------------------------------------------------------------
// LDS read rates: 256-thread workgroups, each filling a 64 KB LDS array and
// then reading it 4096 x 8 times per lane (two workgroups, 8 waves, per CU).
// Kind 0: ds_read_b128, lane l of a wave at 16 l bytes past a per-wave base
// (every 16-lane quarter covers the 64 banks once).  Kind 1:
// ds_read_b64_tr_b16 at the addresses the causal prefill reads its V^T
// operand from (128-dim bf16 rows of 256 bytes, 16-byte chunks permuted by
// XOR with 64 x the 64-dim block; see the prefill kernel), the 8 reads per
// step alternating between two 16 KB halves.  Addresses are precomputed, so
// the loop is the reads and one XOR each.
// ---------------------------------------------------------------------------
namespace {

constexpr int kLdsBytes = 65536;

template <int KIND>
__global__ __launch_bounds__(kThreads) void lds_rate_kernel(uint32_t* sink, uint32_t key) {
  __shared__ __attribute__((aligned(16))) char tile[kLdsBytes];
  for (int i = threadIdx.x; i < kLdsBytes / 16; i += kThreads)
    reinterpret_cast<u32x4_t*>(tile)[i] = u32x4_t{uint32_t(i), 3u * uint32_t(i), 5u, 7u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  if constexpr (KIND == 0) {
    int off = wave * 4096 + lane * 16;
    for (int i = 0; i < kRateSteps; ++i) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        acc ^= *reinterpret_cast<const u32x4_t*>(tile + ((off + u * 1024) & (kLdsBytes - 1)));
      off = (off + 8192) & (kLdsBytes - 1);
    }
  } else {
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    const int l32 = lane & 31, e4 = (l32 >> 2) & 3;
    const int vx = (4 * (lane >> 5) + e4) * 256 + 64 * e4 + 32 * (l32 >> 4) + 8 * (l32 & 3);
    int a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = (vx ^ (64 * (u & 3))) + (u >> 2) * 16 * 256;
    int half = 0;
    for (int i = 0; i < kRateSteps; ++i) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(tile + half + a[u]));
        acc[u & 3] ^= uint32_t(uint16_t(v[0])) ^ (uint32_t(uint16_t(v[1])) << 16) ^ uint32_t(uint16_t(v[2])) ^
                      (uint32_t(uint16_t(v[3])) << 16);
      }
      half ^= 16384;
    }
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == key) sink[0] = 1u;
}

}  // namespace

extern "C" int gqa_probe_lds_rate(uint32_t* sink, int kind, int blocks, void* stream) {
  if (!sink || (reinterpret_cast<uintptr_t>(sink) & 3u) || blocks < 1 || blocks > (1 << 16) || kind < 0 ||
      kind > 1)
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(lds_rate_kernel<0>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, sink, 0x9e3779b9u);
  else
    hipLaunchKernelGGL(lds_rate_kernel<1>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, sink, 0x9e3779b9u);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
