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

// Device-scope (all XCDs) coherent load/store of one word: relaxed atomics at agent
// scope, which go past the per-XCD caches instead of relying on a cache flush.
template <typename T>
__device__ __forceinline__ void coherent_store(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T coherent_load(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same for 16 bytes, through a buffer resource over [base, base + 2 GiB) with the
// agent-scope cache policy (sc1); byte offsets are 32-bit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void coherent_store4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 16);
}
__device__ __forceinline__ f32x4 coherent_load4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16);
}

// acc + lo + hi of a packed bf16 pair (one v_dot2 against (1, 1)).
__device__ __forceinline__ float dot2_ones(uint32_t w, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
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

// Exact OCP E4M3 -> bf16 of two codes (bytes byte0, byte0 + 1 of w; byte0 = 0 or 2):
// every E4M3 value is a bf16 value, and a unit scale leaves it unchanged.
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, int byte0) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = byte0 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}

// Cache code formats (same values as the C ABI's kv_dtype).
enum KvFmt : int { kKvBf16 = 0, kKvInt8 = 1, kKvFp8 = 2, kKvMxfp4 = 3, kKvMxfp8 = 4 };

template <int FMT>
__device__ __forceinline__ uint32_t code2_to_bf16x2(uint32_t w, int byte0) {
  if constexpr (FMT == kKvFp8) return e4m3x2_to_bf16x2(w, byte0);
  else return i8x2_to_bf16x2(w, byte0);
}

// Two codes (bytes byte0, byte0 + 1 of w) times the scale s, each product rounded
// once to fp32 and then to bf16 (nearest even): the dequantised value as bf16.
template <int FMT>
__device__ __forceinline__ uint32_t dequant2_bf16x2(uint32_t w, int byte0, float s) {
  float f0, f1;
  if constexpr (FMT == kKvFp8) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = byte0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true)
                          : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
    f0 = v[0];
    f1 = v[1];
  } else {
    f0 = (float)(int8_t)((w >> (8 * byte0)) & 0xffu);
    f1 = (float)(int8_t)((w >> (8 * (byte0 + 1))) & 0xffu);
  }
  return pack_bf16x2(f0 * s, f1 * s);
}

// Two fp32 values (|y| <= 448) -> two OCP E4M3 codes, round to nearest even, into the
// low (hi_half = false) or high 16 bits of `old`.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float y0, float y1, uint32_t old, bool hi_half) {
  return hi_half ? uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, int(old), true))
                 : uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, int(old), false));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace ll
