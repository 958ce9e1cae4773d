// kvwrite.hip -- write whole frames of K/V into cache slots (append/evict and recache).
//
// Append ("LongLive: Real-time Interactive Long Video Generation" explainer, dpshk.com,
// §二: a finished chunk's K/V enter the cache; §五: frames older than the window are
// evicted) and recache (§三 item 5: the recomputed cache replaces the old one) are the
// same operation here: copy frame i of the caller's tensor into slot plan_slot[i].
// Eviction is the overwrite of a ring slot; no memory is allocated or freed.
//
// bf16 caches: a frame is one contiguous run of T*H*D bf16 in both the source and the
// slot, so this is a streaming 16-byte-vector copy (HBM bound).  Plain loads and
// non-temporal (streaming) stores: measured on gfx950 against the other three
// combinations of the two hints, this one moves the append's 57.5 MB fastest, at the
// speed of the runtime's own device copy of the same bytes; non-temporal loads were
// the slow part.
// int8 caches: each (token, head) row of D values is quantised on the fly
//   a = max |x|, scale = a / 127, q = clamp(rint((x * 127) / a), -127, 127)
// (every operation IEEE binary32, correctly rounded quotient, ties-to-even rounding;
// x * 127 is exact for bf16 x).  fp8 caches: the same with M = 448 (largest finite
// OCP E4M3 value) and the quotient, clamped to [-448, 448] (it exceeds that only when
// x * 448 overflowed), rounded to E4M3 (nearest, ties to even) by the hardware
// conversion.  LongLive-2.0 explainer, wmrh.cn, §15.2: the history cache is
// stored in low precision to save memory and traffic.  MXFP4 / MXFP8 caches: see
// mx_frames_kernel.
#include "device_common.h"
#include "launch.h"

namespace ll {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;      // 16-byte vectors in flight per thread (copies)
constexpr int kQuantRows = 2;     // rows per lane group of the quantising writes
constexpr int kQuantValues = 16;  // values of a row per lane in the quantising writes

// grid: x = block within the frame, y = plan entry, z = 0 (K) / 1 (V)
__global__ __launch_bounds__(kThreads) void copy_frames_kernel(const WriteParams p, int64_t vecs_per_frame) {
  const int e = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const u32x4* src = reinterpret_cast<const u32x4*>(isv ? p.srcV : p.srcK) + int64_t(p.plan_src[e]) * vecs_per_frame;
  u32x4* dst = reinterpret_cast<u32x4*>(isv ? p.dstV : p.dstK) + int64_t(p.plan_slot[e]) * vecs_per_frame;
  const int64_t base = int64_t(blockIdx.x) * (kThreads * kUnroll) + threadIdx.x;
  u32x4 r[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + int64_t(u) * kThreads;
    if (i < vecs_per_frame) r[u] = src[i];
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + int64_t(u) * kThreads;
    if (i < vecs_per_frame) __builtin_nontemporal_store(r[u], dst + i);
  }
}

// Correctly rounded 1/a for a bf16 value a (8-bit significand) in the normal range: the
// hardware reciprocal (within 1 ulp) and one Newton step with FMAs.  The step leaves a
// relative error below 2^-45, and 1/a for an 8-bit significand lies at least 2^-25
// (relative) away from any midpoint between binary32 neighbours (or is exact), so the
// final rounding gives RN(1/a).  (Checked on gfx950 against IEEE division for every bf16
// absmax in [2^-100, 2^120].)
__device__ __forceinline__ float rcp_rn_bf16(float a) {
  const float y0 = __builtin_amdgcn_rcpf(a);
  const float e = __builtin_fmaf(-a, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}

// RN(a / M) by Markstein's correction with the constant RN(1/M) (valid without overflow
// or underflow; the same check as above).
template <int FMT>
__device__ __forceinline__ float div_by_M(float a) {
  constexpr float M = FMT == kKvFp8 ? 448.0f : 127.0f;
  constexpr float yM = 1.0f / M;
  const float q0 = a * yM;
  const float r = __builtin_fmaf(-M, q0, a);
  return __builtin_fmaf(r, yM, q0);
}

// Max over the LPR (4, 8 or 16) lanes of a row, every lane ends with it: DPP inside quads
// (xor 1, xor 2), then the half-row (8 lanes) and row (16 lanes) mirrors.
template <int LPR>
__device__ __forceinline__ float row_max(float v) {
  auto dpp = [](float x, int ctrl) __attribute__((always_inline)) {
    switch (ctrl) {
      case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
      case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
      case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
      default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    }
  };
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "rows of 4, 8 or 16 lanes");
  v = fmaxf(v, dpp(v, 0xB1));
  v = fmaxf(v, dpp(v, 0x4E));
  if constexpr (LPR >= 8) v = fmaxf(v, dpp(v, 0x141));
  if constexpr (LPR == 16) v = fmaxf(v, dpp(v, 0x140));
  return v;
}

// One (token, head) row of D values per LPR = D / 16 lanes (aligned to DPP rows); each
// lane owns 16 consecutive values of RPG rows (two 16-byte loads each, all issued before
// any arithmetic) and stores their 16 codes with one 16-byte store.
//
// Division: q = rint(n / a) with n = x * M needs the correctly rounded quotient.  With
// y = RN(1/a) and q0 = RN(n * y) within one ulp of n/a, the residual r = n - a * q0 is
// exact as one FMA and RN(q0 + r * y) is the correctly rounded n/a (Markstein's theorem
// for floating-point division, e.g. J.-M. Muller et al., Handbook of Floating-Point
// Arithmetic, ch. on division).  It needs no underflow or overflow, so rows whose
// absmax is below 2^-100 or above 2^120 (where x * M may overflow) take plain IEEE
// divisions and the clamp; everywhere else |n / a| <= M holds exactly.
// int8 codes: |q| <= 127, so q + 1.5 * 2^23 lies in [2^23, 2^24), where the spacing of
// binary32 is 1: that one addition rounds q to the nearest integer, ties to even (rint),
// and leaves it in the low byte of the sum's bits as a two's-complement byte.
template <int D, int FMT>
__global__ __launch_bounds__(kThreads) void quant_frames_kernel(const WriteParams p) {
  constexpr float M = FMT == kKvFp8 ? 448.0f : 127.0f;
  constexpr int VPL = kQuantValues;
  constexpr int LPR = D / VPL;
  constexpr int GROUPS = kThreads / LPR;
  constexpr int RPG = kQuantRows;
  const int e = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const int sub = threadIdx.x % LPR;
  const int64_t row0 = (int64_t(blockIdx.x) * GROUPS + threadIdx.x / LPR) * RPG;
  const uint16_t* src = (isv ? p.srcV : p.srcK) + int64_t(p.plan_src[e]) * p.rows_per_frame * D;
  int8_t* dst = static_cast<int8_t*>(isv ? p.dstV : p.dstK) + int64_t(p.plan_slot[e]) * p.rows_per_frame * D;
  float* dsc = (isv ? p.dstVs : p.dstKs) + int64_t(p.plan_slot[e]) * p.rows_per_frame;

  u32x4 w[RPG][VPL / 8];
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    const int64_t row = row0 + rr;
#pragma unroll
    for (int h = 0; h < VPL / 8; ++h)
      w[rr][h] = row < p.rows_per_frame ? *reinterpret_cast<const u32x4*>(src + row * D + VPL * sub + 8 * h)
                                        : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    const int64_t row = row0 + rr;
    float x[VPL];
#pragma unroll
    for (int h = 0; h < VPL / 8; ++h)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * h + 2 * k] = __builtin_bit_cast(float, w[rr][h][k] << 16);
        x[8 * h + 2 * k + 1] = __builtin_bit_cast(float, w[rr][h][k] & 0xffff0000u);
      }
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) a = fmaxf(a, fabsf(x[k]));
    a = row_max<LPR>(a);

    float scale = 0.0f;
    uint32_t packed[VPL / 4] = {};
    auto pack = [&](const float (&qq)[VPL]) __attribute__((always_inline)) {
      if constexpr (FMT == kKvFp8) {
#pragma unroll
        for (int w2 = 0; w2 < VPL / 4; ++w2) {
          packed[w2] = f32x2_to_e4m3x2(__builtin_copysignf(qq[4 * w2], x[4 * w2]),
                                       __builtin_copysignf(qq[4 * w2 + 1], x[4 * w2 + 1]), 0u, false);
          packed[w2] = f32x2_to_e4m3x2(__builtin_copysignf(qq[4 * w2 + 2], x[4 * w2 + 2]),
                                       __builtin_copysignf(qq[4 * w2 + 3], x[4 * w2 + 3]), packed[w2], true);
        }
      } else {
        uint32_t t[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) t[k] = __builtin_bit_cast(uint32_t, qq[k] + 12582912.0f);
#pragma unroll
        for (int j = 0; j < VPL / 4; ++j)
          packed[j] = __builtin_amdgcn_perm(t[4 * j + 1], t[4 * j], 0x0c0c0400u) |
                      __builtin_amdgcn_perm(t[4 * j + 3], t[4 * j + 2], 0x04000c0cu);
      }
    };
    // Rows whose absmax is zero or outside [2^-100, 2^120] take plain divisions; the
    // test is made once per wave, so that the common case runs without a branch per
    // value (the per-lane form compiled to an exec-masked branch around each value).
    const bool plain = !(a >= 0x1p-100f && a <= 0x1p+120f);
    if (__builtin_amdgcn_ballot_w64(plain) == 0) {
      scale = div_by_M<FMT>(a);
      const float y = rcp_rn_bf16(a);
      float qq[VPL];
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        const float n = x[k] * M;   // exact for bf16 x
        const float q0 = n * y;
        const float r = __builtin_fmaf(-a, q0, n);
        qq[k] = __builtin_fmaf(r, y, q0);
      }
      pack(qq);
    } else if (a > 0.0f) {
      const bool pl = a < 0x1p-100f || a > 0x1p+120f;
      scale = pl ? a / M : div_by_M<FMT>(a);
      const float y = pl ? 1.0f / a : rcp_rn_bf16(a);
      float qq[VPL];
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        const float n = x[k] * M;   // exact for bf16 x unless it overflows
        if (pl) {
          qq[k] = fminf(fmaxf(n / a, -M), M);
        } else {
          qq[k] = n * y;
          const float r = __builtin_fmaf(-a, qq[k], n);
          qq[k] = __builtin_fmaf(r, y, qq[k]);
        }
      }
      pack(qq);
    }
    if (row < p.rows_per_frame) {
#pragma unroll
      for (int h = 0; h < VPL / 16; ++h)
        __builtin_nontemporal_store(u32x4{packed[4 * h], packed[4 * h + 1], packed[4 * h + 2], packed[4 * h + 3]},
                                    reinterpret_cast<u32x4*>(dst + row * D + VPL * sub + 16 * h));
      if (sub == 0) dsc[row] = scale;
    }
  }
}

// MX caches (OCP Microscaling: one E8M0 power-of-two scale per block of 32 values;
// elements E2M1 for MXFP4, E4M3 for MXFP8; LongLive-2.0 explainer, wmrh.cn, §15.2: the
// history cache in low-precision floating point).  Same lane layout as the quantising
// writes above: D/16 lanes per (token, head) row, 16 consecutive values per lane, so a
// block of 32 is a lane pair.  Per block: a = max |x| (lane pair, one DPP swap),
// e = max(floor(log2 a) - EMAX, EMIN) read off a's exponent field (a bf16 value; 0 and
// subnormals give EMIN), y = x * 2^-e (exact), and the hardware conversion with unit
// scale: nearest, ties to the even code, sign kept (E2M1 saturates at 6 by itself;
// E4M3 values are clamped to +-448 first).  Both conversions were checked against the
// formats' definitions (midpoints, saturation, signed zeros).  A lane's 16 codes leave
// with one 8-byte (MXFP4, value 2k in the low half of byte k) or 16-byte (MXFP8) store;
// the first lane of a row gathers the row's block exponents into one scale word (byte
// b = e_b + 127).
template <int D, int FMT>
__global__ __launch_bounds__(kThreads) void mx_frames_kernel(const WriteParams p) {
  constexpr bool FP4 = FMT == kKvMxfp4;
  constexpr int EMAX = FP4 ? 2 : 8;        // exponent of the element format's largest value
  constexpr int EMIN = FP4 ? -125 : -117;  // smallest value * 2^EMIN is 2^-126, a normal bf16
  constexpr int RB = FP4 ? D / 2 : D;      // code bytes per row
  constexpr int VPL = kQuantValues;
  constexpr int LPR = D / VPL;
  constexpr int GROUPS = kThreads / LPR;
  constexpr int RPG = kQuantRows;
  static_assert(VPL == 16 && (LPR == 4 || LPR == 8), "a block of 32 values is a lane pair");
  const int e = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const int sub = threadIdx.x % LPR;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = (int64_t(blockIdx.x) * GROUPS + threadIdx.x / LPR) * RPG;
  const uint16_t* src = (isv ? p.srcV : p.srcK) + int64_t(p.plan_src[e]) * p.rows_per_frame * D;
  uint8_t* dst = static_cast<uint8_t*>(isv ? p.dstV : p.dstK) + int64_t(p.plan_slot[e]) * p.rows_per_frame * RB;
  uint32_t* dsc = reinterpret_cast<uint32_t*>(isv ? p.dstVs : p.dstKs) + int64_t(p.plan_slot[e]) * p.rows_per_frame;

  u32x4 w[RPG][VPL / 8];
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    const int64_t row = row0 + rr;
#pragma unroll
    for (int h = 0; h < VPL / 8; ++h)
      w[rr][h] = row < p.rows_per_frame ? *reinterpret_cast<const u32x4*>(src + row * D + VPL * sub + 8 * h)
                                        : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    const int64_t row = row0 + rr;
    float x[VPL];
#pragma unroll
    for (int h = 0; h < VPL / 8; ++h)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * h + 2 * k] = __builtin_bit_cast(float, w[rr][h][k] << 16);
        x[8 * h + 2 * k + 1] = __builtin_bit_cast(float, w[rr][h][k] & 0xffff0000u);
      }
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) a = fmaxf(a, fabsf(x[k]));
    a = fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, false)));
    const int eb = max(int(__builtin_bit_cast(uint32_t, a) >> 23) - 127 - EMAX, EMIN);
    const float inv = __builtin_bit_cast(float, uint32_t(127 - eb) << 23);   // 2^-e, a normal float
    uint32_t c[4] = {0u, 0u, 0u, 0u};
    if constexpr (FP4) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        c[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[h], x[8 * h] * inv, x[8 * h + 1] * inv, 1.0f, 0);
        c[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[h], x[8 * h + 2] * inv, x[8 * h + 3] * inv, 1.0f, 1);
        c[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[h], x[8 * h + 4] * inv, x[8 * h + 5] * inv, 1.0f, 2);
        c[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[h], x[8 * h + 6] * inv, x[8 * h + 7] * inv, 1.0f, 3);
      }
    } else {
      float y[VPL];
#pragma unroll
      for (int k = 0; k < VPL; ++k) y[k] = fminf(fmaxf(x[k] * inv, -448.0f), 448.0f);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        c[h] = f32x2_to_e4m3x2(y[4 * h], y[4 * h + 1], 0u, false);
        c[h] = f32x2_to_e4m3x2(y[4 * h + 2], y[4 * h + 3], c[h], true);
      }
    }
    // scale word of the row: block b's byte comes from lane sub = 2 b of the row
    const int byte = eb + 127;
    uint32_t word = uint32_t(byte);
#pragma unroll
    for (int b = 1; b < D / 32; ++b)
      word |= uint32_t(__builtin_amdgcn_ds_bpermute(4 * ((lane + 2 * b) & 63), byte)) << (8 * b);
    if (row < p.rows_per_frame) {
      if constexpr (FP4) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u32x2{c[0], c[1]}, reinterpret_cast<u32x2*>(dst + row * RB + 8 * sub));
      } else {
        __builtin_nontemporal_store(u32x4{c[0], c[1], c[2], c[3]}, reinterpret_cast<u32x4*>(dst + row * RB + 16 * sub));
      }
      if (sub == 0) dsc[row] = word;
    }
  }
}

}  // namespace

hipError_t launch_kv_write(const WriteParams& p, int D, int kv_fmt, hipStream_t s) {
  if (p.n <= 0) return hipSuccess;
  if (kv_fmt == kKvBf16) {
    const int64_t vecs = p.rows_per_frame * D * 2 / 16;
    const int64_t per_block = int64_t(kThreads) * kUnroll;
    dim3 grid(unsigned((vecs + per_block - 1) / per_block), unsigned(p.n), 2);
    hipLaunchKernelGGL(copy_frames_kernel, grid, dim3(kThreads), 0, s, p, vecs);
    return hipGetLastError();
  }
  const int rows_per_block = kThreads / (D / kQuantValues) * kQuantRows;
  dim3 grid(unsigned((p.rows_per_frame + rows_per_block - 1) / rows_per_block), unsigned(p.n), 2);
  if (kv_fmt == kKvMxfp4 || kv_fmt == kKvMxfp8) {
    if (D == 128 && kv_fmt == kKvMxfp4) hipLaunchKernelGGL((mx_frames_kernel<128, kKvMxfp4>), grid, dim3(kThreads), 0, s, p);
    else if (D == 64 && kv_fmt == kKvMxfp4) hipLaunchKernelGGL((mx_frames_kernel<64, kKvMxfp4>), grid, dim3(kThreads), 0, s, p);
    else if (D == 128) hipLaunchKernelGGL((mx_frames_kernel<128, kKvMxfp8>), grid, dim3(kThreads), 0, s, p);
    else if (D == 64) hipLaunchKernelGGL((mx_frames_kernel<64, kKvMxfp8>), grid, dim3(kThreads), 0, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (D == 128 && kv_fmt == kKvInt8) hipLaunchKernelGGL((quant_frames_kernel<128, kKvInt8>), grid, dim3(kThreads), 0, s, p);
  else if (D == 64 && kv_fmt == kKvInt8) hipLaunchKernelGGL((quant_frames_kernel<64, kKvInt8>), grid, dim3(kThreads), 0, s, p);
  else if (D == 128 && kv_fmt == kKvFp8) hipLaunchKernelGGL((quant_frames_kernel<128, kKvFp8>), grid, dim3(kThreads), 0, s, p);
  else if (D == 64 && kv_fmt == kKvFp8) hipLaunchKernelGGL((quant_frames_kernel<64, kKvFp8>), grid, dim3(kThreads), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ll
