// Device helpers shared by the gfx950 kernels: bf16 bit conversions, MFMA
// operand types and 64-lane cross-lane moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 is the upper half of a binary32 word: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Value of lane (16 * (lane / 16) + N) in every lane of its 16-lane row
// (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, 0x150 + N, 0xf, 0xf, false);
}

__device__ __forceinline__ float read_lane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ int uniform_int(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Sum / max over the lane pairs (l, l ^ 16) and (l, l ^ 32), with the gfx950
// row-swap moves: permlane16_swap exchanges odd 16-lane rows of one operand
// with even rows of the other, permlane32_swap the two 32-lane halves, so
// swapping a value with itself puts both partners of every pair side by side.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace pkv
