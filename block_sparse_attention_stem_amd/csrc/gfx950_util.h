// gfx950 (CDNA4) building blocks: vector types for the MFMA operands, raw
// 16-byte loads/stores, and the lane-layout facts the kernels rely on.
//
// MFMA 32x32 output layout (v_mfma_f32_32x32x16_bf16 and the 32x32x64 fp8
// form): lane l holds column n = l % 32 and, in accumulator register i
// (0..15), row m = 8*(i/4) + 4*(l/32) + (i%4).  The A operand gives row
// m = l % 32 and the B operand column n = l % 32; both take their k-slots
// from lane group l / 32 with the same slot-to-k map, so any permutation of
// k that is applied identically to A and B leaves the product unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stem {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8;

__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
__device__ __forceinline__ void st8(void *p, u32x2 v) { *reinterpret_cast<u32x2 *>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f16_32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// fp8 (OCP e4m3fn) x fp8 -> fp32, 32x32x64.  Format code 0 selects e4m3 for
// both operands; the E8M0 block scales are 127 (= 2^0), i.e. unscaled.
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Round-to-nearest-even fp32 pair -> packed bf16x2 (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Round-to-nearest-even fp32 pair -> packed fp16x2 (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Two bf16 values (lo, hi halves) -> the same two values as fp16.  Exact for
// magnitudes in [2^-14, 65504] (every bf16 significand fits in fp16's);
// smaller ones keep 2^-24 absolute resolution and larger ones saturate to
// +-65504 (round toward zero never produces inf from a finite input).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  const float lo = __uint_as_float(x << 16), hi = __uint_as_float(x & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Byte/half selection: result byte k = byte sel_k of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ float wave_max_xor32(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}

}  // namespace stem
