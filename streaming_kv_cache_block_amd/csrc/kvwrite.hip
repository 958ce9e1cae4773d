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
// stored in low precision to save memory and traffic.
#include "device_common.h"
#include "launch.h"

namespace ll {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte vectors in flight per thread

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

// One (token, head) row of D values per LPR = D / 8 lanes; each lane owns 8 values of
// RPG rows, whose loads are all issued before any arithmetic (bytes in flight).
//
// Division: q = rint(n / a) with n = x * 127 needs the correctly rounded quotient.  With
// y = RN(1/a) (one IEEE division per row) and q0 = RN(n * y) within one ulp of n/a, the
// residual r = n - a * q0 is exact as one FMA and RN(q0 + r * y) is the correctly rounded
// n/a (Markstein's theorem for floating-point division, e.g. J.-M. Muller et al.,
// Handbook of Floating-Point Arithmetic, ch. on division).  It needs no underflow or
// overflow, so rows whose absmax is below 2^-100 or above 2^120 (where x * 127 may
// overflow) use the plain IEEE division.
template <int D, int FMT>
__global__ __launch_bounds__(kThreads) void quant_frames_kernel(const WriteParams p) {
  constexpr float M = FMT == kKvFp8 ? 448.0f : 127.0f;
  constexpr int LPR = D / 8;
  constexpr int GROUPS = kThreads / LPR;
  constexpr int RPG = 4;
  const int e = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const int sub = threadIdx.x % LPR;
  const int64_t row0 = (int64_t(blockIdx.x) * GROUPS + threadIdx.x / LPR) * RPG;
  const uint16_t* src = (isv ? p.srcV : p.srcK) + int64_t(p.plan_src[e]) * p.rows_per_frame * D;
  int8_t* dst = static_cast<int8_t*>(isv ? p.dstV : p.dstK) + int64_t(p.plan_slot[e]) * p.rows_per_frame * D;
  float* dsc = (isv ? p.dstVs : p.dstKs) + int64_t(p.plan_slot[e]) * p.rows_per_frame;

  u32x4 w[RPG];
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    const int64_t row = row0 + rr;
    w[rr] = row < p.rows_per_frame ? *reinterpret_cast<const u32x4*>(src + row * D + 8 * sub)
                                   : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    const int64_t row = row0 + rr;
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __builtin_bit_cast(float, w[rr][k] << 16);
      x[2 * k + 1] = __builtin_bit_cast(float, w[rr][k] & 0xffff0000u);
    }
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(x[k]));
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, LPR));

    const float scale = a / M;
    uint32_t packed[2] = {0u, 0u};
    if (a > 0.0f) {
      const bool plain = a < 0x1p-100f || a > 0x1p+120f;
      const float y = 1.0f / a;
      float qq[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float n = x[k] * M;   // exact for bf16 x
        if (plain) {
          qq[k] = n / a;
        } else {
          qq[k] = n * y;
          const float r = __builtin_fmaf(-a, qq[k], n);
          qq[k] = __builtin_fmaf(r, y, qq[k]);
        }
      }
      if constexpr (FMT == kKvFp8) {
        // |quotient| <= 448 except when x * 448 overflowed (inf): saturate like the clamp.
        // The FMA correction turns a -0 quotient into +0; the IEEE quotient has the sign
        // of x (a > 0), and E4M3 keeps the sign of zero.
#pragma unroll
        for (int k = 0; k < 8; ++k) qq[k] = __builtin_copysignf(fminf(fmaxf(qq[k], -448.0f), 448.0f), x[k]);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          packed[w] = f32x2_to_e4m3x2(qq[4 * w], qq[4 * w + 1], 0u, false);
          packed[w] = f32x2_to_e4m3x2(qq[4 * w + 2], qq[4 * w + 3], packed[w], true);
        }
      } else {
        // q = clamp(rint(quotient), -127, 127) is an integer, so q + 128 in [1, 255] is
        // exact and converts exactly to an unsigned byte; flipping bit 7 of each byte
        // then gives the two's-complement code of q.
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float t = __builtin_amdgcn_fmed3f(__builtin_rintf(qq[k]), -127.0f, 127.0f) + 128.0f;
          packed[k >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(t, k & 3, packed[k >> 2]);
        }
        packed[0] ^= 0x80808080u;
        packed[1] ^= 0x80808080u;
      }
    }
    if (row < p.rows_per_frame) {
      __builtin_nontemporal_store(u32x2{packed[0], packed[1]}, reinterpret_cast<u32x2*>(dst + row * D + 8 * sub));
      if (sub == 0) dsc[row] = scale;   // 4-byte scales of adjacent rows merge in the L2
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
  const int rows_per_block = kThreads / (D / 8) * 4;
  dim3 grid(unsigned((p.rows_per_frame + rows_per_block - 1) / rows_per_block), unsigned(p.n), 2);
  if (D == 128 && kv_fmt == kKvInt8) hipLaunchKernelGGL((quant_frames_kernel<128, kKvInt8>), grid, dim3(kThreads), 0, s, p);
  else if (D == 64 && kv_fmt == kKvInt8) hipLaunchKernelGGL((quant_frames_kernel<64, kKvInt8>), grid, dim3(kThreads), 0, s, p);
  else if (D == 128 && kv_fmt == kKvFp8) hipLaunchKernelGGL((quant_frames_kernel<128, kKvFp8>), grid, dim3(kThreads), 0, s, p);
  else if (D == 64 && kv_fmt == kKvFp8) hipLaunchKernelGGL((quant_frames_kernel<64, kKvFp8>), grid, dim3(kThreads), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ll
