// device_common.h -- gfx950 vector types and small device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ll {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Wave64 32x32x16 bf16 MFMA, fp32 accumulate (gfx950).
//   A: lane l holds row (l % 32), k = 8*(l / 32) + [0, 8)
//   B: lane l holds column (l % 32), k = 8*(l / 32) + [0, 8)
//   C: lane l holds column (l % 32), rows 8*i + 4*(l / 32) + j at element 4*i + j
// Only the A/B pairing of k matters for the result: any k order that A and B share
// gives the same sum.
__device__ __forceinline__ f32x16 mfma32(const bf16x8 a, const bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Select 16-bit halves: result = (b.half[hb] << 16) | a.half[ha].
__device__ __forceinline__ uint32_t pick_lo_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pick_hi_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Exact int8 -> bf16 for |q| <= 127: the fp32 value has at most 7 significant bits,
// so its upper 16 bits are the bf16 encoding.
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int byte0) {
  float f0 = (float)(int8_t)((w >> (8 * byte0)) & 0xffu);
  float f1 = (float)(int8_t)((w >> (8 * (byte0 + 1))) & 0xffu);
  return pick_hi_hi(__builtin_bit_cast(uint32_t, f0), __builtin_bit_cast(uint32_t, f1));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace ll
