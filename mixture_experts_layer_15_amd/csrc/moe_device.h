// Device-side helpers shared by the gfx950 kernels: storage formats, MFMA
// operand types and wavefront utilities.  Wave size is 64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // one 16-byte chunk
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bfloat16 is stored as its 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest even (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// Four OCP E4M3FN codes (one dword) -> four bfloat16 (two dwords), exactly:
// every finite E4M3FN value has at most 4 significant bits and an exponent
// inside bfloat16's normal range, so the conversion with unit scale rounds
// nothing.
__device__ __forceinline__ u32x2_t e4m3x4_to_bf16x4(uint32_t q) {
  bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, false);
  bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, true);
  return u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// One E8M0 scale byte -> its float32 value 2^(s - 127) (s = 0 is the
// float32 subnormal 2^-127; s = 255, NaN in the format, is outside the
// library's contract).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Eight OCP E2M1 codes (one dword, element 2j in the low nibble of byte j)
// times a power-of-two scale -> eight bfloat16.  Exact: an E2M1 value has at
// most 2 significant bits, so every product with a scale in 2^-127 .. 2^125
// is a bfloat16 (v_cvt_scalef32_pk_bf16_fp4, one byte per instruction).
__device__ __forceinline__ bf16x8_t e2m1x8_to_bf16x8(uint32_t q, float scale) {
  const bf16x2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
  const bf16x2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1);
  const bf16x2_t b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2);
  const bf16x2_t b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3);
  return __builtin_bit_cast(bf16x8_t, u32x4_t{__builtin_bit_cast(uint32_t, b0),
                                              __builtin_bit_cast(uint32_t, b1),
                                              __builtin_bit_cast(uint32_t, b2),
                                              __builtin_bit_cast(uint32_t, b3)});
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave-wide sum with a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// silu(z) = z * sigmoid(z) with the hardware exp2 and reciprocal (about 1 ulp
// each; the bf16/fp8 paths round h to bf16 right after).
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

}  // namespace moe
