// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Two floats -> two bfloat16 (round to nearest even), packed lo | hi << 16.
// gfx950 has a packed conversion instruction for this.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  bf16x2_t r = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return uint16_t(pack_bf16x2(x, 0.f) & 0xffffu);
}

// 16-byte global load / store.
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
// 16-byte load of data read once (non-temporal hint: streams past the caches).
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

// Cross-lane helpers over a wave of 64.
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

template <int WIDTH>
__device__ __forceinline__ float reduce_sum_lanes(float v) {
  // butterfly over lanes whose index differs in the low log2(WIDTH) bits
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) v += shfl_xor(v, m);
  return v;
}

// Compiler barrier plus a wait for this wave's outstanding LDS operations.
__device__ __forceinline__ void lds_wave_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

}  // namespace gqa
