// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
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

// IEEE half: two floats -> two halves (round to nearest even), and back.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  f16x2_t r = __builtin_convertvector(f, f16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float f16lo_to_f32(uint32_t w) {
  return float(__builtin_bit_cast(f16x2_t, w)[0]);
}
__device__ __forceinline__ float f16hi_to_f32(uint32_t w) {
  return float(__builtin_bit_cast(f16x2_t, w)[1]);
}
__device__ __forceinline__ uint16_t to_f16(float x) {
  return uint16_t(pack_f16x2(x, 0.f) & 0xffffu);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return float(__builtin_bit_cast(_Float16, h));
}

// The two 16-bit element formats of the matrix-core paths, selected by the
// dtype code (1 = bfloat16, 2 = IEEE half): packing of float pairs (round to
// nearest even), unpacking, and the sum of a packed pair in float32.
template <int DT>
struct Half16;
template <>
struct Half16<1> {
  __device__ static uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
  __device__ static float lo(uint32_t w) { return bf16lo_to_f32(w); }
  __device__ static float hi(uint32_t w) { return bf16hi_to_f32(w); }
  __device__ static float sum2(uint32_t w, float acc) {   // acc + lo + hi (one dot2)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
  }
};
template <>
struct Half16<2> {
  __device__ static uint32_t pack2(float lo, float hi) { return pack_f16x2(lo, hi); }
  __device__ static float lo(uint32_t w) { return f16lo_to_f32(w); }
  __device__ static float hi(uint32_t w) { return f16hi_to_f32(w); }
  __device__ static float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), __builtin_bit_cast(f16x2_t, 0x3c003c00u),
                                  acc, false);
  }
};

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

// Sum over aligned groups of WIDTH lanes (1 .. 64), every lane of a group
// receiving the group's sum, without the LDS crossbar: DPP quad permutations
// (lane ^ 1, lane ^ 2), the half-row and row mirrors (after the quad steps
// every lane of a quad holds the quad's sum, so the mirror partner holds the
// other quad's or half-row's), then gfx950's row-swap instructions for 32 and
// 64 lanes.  Float addition is commutative, so every lane of a group ends with
// the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int WIDTH>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (WIDTH >= 2) v += dpp_mov<0xB1>(v);     // quad_perm [1,0,3,2]
  if constexpr (WIDTH >= 4) v += dpp_mov<0x4E>(v);     // quad_perm [2,3,0,1]
  if constexpr (WIDTH >= 8) v += dpp_mov<0x141>(v);    // row_half_mirror
  if constexpr (WIDTH >= 16) v += dpp_mov<0x140>(v);   // row_mirror
  if constexpr (WIDTH >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (WIDTH >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

// Maximum over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48),
// every lane receiving it, with gfx950's row-swap instructions.
__device__ __forceinline__ float max_over_rows(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

// Compiler barrier plus a wait for this wave's outstanding LDS operations.
__device__ __forceinline__ void lds_wave_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

}  // namespace gqa
