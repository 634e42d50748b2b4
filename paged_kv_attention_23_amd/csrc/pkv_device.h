// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, the 16x16x32 bf16 matrix-core instruction and wave shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16).  Lane l supplies row (l % 16)
// of A and column (l % 16) of B, each as 8 consecutive k-elements of k-group
// l / 16; lane l receives D rows 4*(l/16)+0..3 of column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Round two floats to bf16 (nearest-even, hardware v_cvt_pk_bf16_f32) and pack.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// Cross-row butterfly steps on the gfx950 lane-swap instructions.  Swapping a
// register with itself returns, per lane, the pair {own value, value of lane
// l ^ 16} (permlane16_swap) or {own, lane l ^ 32} (permlane32_swap) in some
// order, so a symmetric combine of the pair is the xor-16 / xor-32 step.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// gfx950 transposing LDS read of 64 bits per lane (four 16-bit values).
// Within each group of 16 lanes, with lane s addressing four consecutive
// values D[s][0..3], lane i receives D[4*j + i/4][i%4] for j = 0..3: if lane s
// addresses key row k0 + s/4 at column c(s%4), lane i receives column
// c(i/4) + i%4 of the four rows k0..k0+3, a column operand for the matrix
// cores.  The address must be 8-byte aligned.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const char *p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)const_cast<char *>(p));
  return __builtin_bit_cast(u32x2, r);
}

}  // namespace pkv
