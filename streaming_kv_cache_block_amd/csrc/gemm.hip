// gemm.hip -- recache projection K_all = h W_K^T, V_all = h W_V^T (bf16 MFMA, fp32 sums).
//
// "LongLive: Real-time Interactive Long Video Generation" explainer, dpshk.com, §三
// item 4: self-attention keys and values are projections of the prompt-conditioned
// hidden state, K = W_K h', V = W_V h'; item 5: recache recomputes them for the
// retained latents under the new prompt.  W is the [d_out][d_in] matrix of that
// column form, so both operands are contiguous along the contraction d_in.
//
// Tiling: a workgroup of 4 waves computes 256 tokens x 128 outputs; each wave 128
// tokens x 64 outputs with 32x32x16 bf16 MFMAs (W rows as the A operand, h rows as
// the B operand, so a lane's accumulators hold 4 consecutive outputs of one token and
// the bf16 results leave as 8-byte stores).  The contraction is walked in steps of 32:
// each step's h and W tiles are copied global -> LDS with the load-to-LDS path into
// two buffers that are separate LDS objects (buffer parity fixed at compile time, so
// the copy of step s+1 overlaps the MFMAs of step s).  Within a 64-byte row the four
// 16-byte chunks are XOR-swizzled by (row >> 2) & 3, which makes the 16 rows that one
// operand read touches land on 16 distinct bank groups.  48 KB of LDS and <= 256
// registers let two workgroups share a CU (two waves per SIMD).  blockIdx.z selects
// the K or V projection, and workgroups that share an h tile run on the same XCD.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ll {
namespace {

constexpr int TM = 256;      // tokens per workgroup
constexpr int TN = 128;      // outputs per workgroup
constexpr int TK = 32;       // contraction step
constexpr int NT = 256;
constexpr int NXCD = 8;
constexpr int HCOPY = TM * TK * 2 / 1024;   // 1 KB wave-wide copies of the h tile (16)
constexpr int WCOPY = TN * TK * 2 / 1024;   // of the W tile (8)

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// element offset of 16-byte chunk c (0..3) of row r in a swizzled [rows][TK] tile
__device__ __forceinline__ int gswz(int r, int c) { return r * TK + 8 * (c ^ ((r >> 2) & 3)); }

// Copy rows [0, rows) x [k0, k0 + TK) of a row-major [*, ld] bf16 matrix into LDS.
// Lane l of copy i fills LDS bytes [1 KB i + 16 l, +16): row 16 i + l / 4, chunk
// position l % 4, which holds source chunk (l % 4) ^ ((row >> 2) & 3).
template <int NCOPY>
__device__ __forceinline__ void copy_tile(const uint16_t* g, int64_t ld, int row0, int rows_valid, int k0,
                                          uint16_t* lds, int wave, int lane) {
#pragma unroll
  for (int i = wave; i < NCOPY; i += 4) {
    const int r = 16 * i + lane / 4;
    const int c = (lane % 4) ^ ((r >> 2) & 3);
    const int rr = min(r, rows_valid - 1);
    __builtin_amdgcn_global_load_lds((gbl_void*)(g + int64_t(row0 + rr) * ld + k0 + 8 * c),
                                     (lds_void*)(lds + 16 * i * TK), 16, 0, 0);
  }
}

// Row of the cache slot array that output row m lands in: frame m / T goes to slot
// plan[m / T] (plan in LDS), token m % T; -1 when the plan has no slot there.
__device__ __forceinline__ int64_t slot_row(int m, int T, const int* plan) {
  const int s = plan[m / T];
  return s < 0 ? -1 : int64_t(s) * T + m % T;
}

// Epilogue of the fused recache: bf16 results, or their int8 / fp8 quantisation
//   a = max |x| over the (token, head) row, scale = a / M,
//   q = clamp(rint((x * M) / a), -M, M) with M = 127   (0 for an all-zero row),
//   or the E4M3 rounding of clamp((x * M) / a, -M, M) with M = 448,
// with the quotient correctly rounded as in the int8 cache writer (one IEEE reciprocal
// per row and a Markstein FMA correction; plain division where the absmax is below
// 2^-100 or above 2^120).  x is the bf16-rounded sum, exactly what a separate
// projection would have stored.
template <int EPI>
__device__ __forceinline__ void cache_epilogue(const ProjToCacheParams& pc, const f32x16 (&acc)[2][4], int m0, int n0,
                                               int z, int wm, int wn, int g, int r32, int tid) {
  // A frame may be held by two slots (a shot-sink frame still in the window): the row
  // is then written to both.
  __shared__ int plan[kMaxPlan], plan2[kMaxPlan];
  __shared__ float amax[2][2][128];   // [wm][wn][token within the wave's half]
  const ProjParams& p = pc.proj;
  for (int i = tid; i < pc.n_plan; i += NT) {
    plan[i] = pc.plan_slot[i];
    plan2[i] = pc.plan_slot2[i];
  }
  __syncthreads();
  const int N = p.N;
  if constexpr (EPI == 1) {
    uint16_t* base = static_cast<uint16_t*>(z ? pc.slotV : pc.slotK);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = m0 + 128 * wm + 32 * b + r32;
      if (row >= p.M) continue;
      const int64_t r2 = slot_row(row, pc.T, plan2);
      uint16_t* dst = base + slot_row(row, pc.T, plan) * N + n0 + 64 * wn;
      uint16_t* dst2 = base + (r2 < 0 ? 0 : r2) * N + n0 + 64 * wn;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 w;
          w.x = pack_bf16x2(acc[a][b][4 * i + 0], acc[a][b][4 * i + 1]);
          w.y = pack_bf16x2(acc[a][b][4 * i + 2], acc[a][b][4 * i + 3]);
          *reinterpret_cast<u32x2*>(dst + 32 * a + 8 * i + 4 * g) = w;
          if (r2 >= 0) *reinterpret_cast<u32x2*>(dst2 + 32 * a + 8 * i + 4 * g) = w;
        }
    }
  } else {
    // bf16-round, then the absmax of each (token, head) row: 32 values per lane, lanes
    // g = 0/1 hold a wave's 64 outputs; with D = 128 the two output-half waves combine
    // through LDS, with D = 64 a wave's 64 outputs are one head.
    float x[4][2][16];
    float am[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float mx = 0.0f;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t bits = pack_bf16x2(acc[a][b][v], 0.0f) << 16;
          x[b][a][v] = __builtin_bit_cast(float, bits);
          mx = fmaxf(mx, fabsf(x[b][a][v]));
        }
      am[b] = fmaxf(mx, __shfl_xor(mx, 32));
    }
    if (pc.D == 128) {
      if (g == 0) {
#pragma unroll
        for (int b = 0; b < 4; ++b) amax[wm][wn][32 * b + r32] = am[b];
      }
      __syncthreads();
#pragma unroll
      for (int b = 0; b < 4; ++b) am[b] = fmaxf(am[b], amax[wm][wn ^ 1][32 * b + r32]);
    }
    constexpr float QM = EPI == 3 ? 448.0f : 127.0f;
    int8_t* base = static_cast<int8_t*>(z ? pc.slotV : pc.slotK);
    float* sc = z ? pc.scV : pc.scK;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = m0 + 128 * wm + 32 * b + r32;
      if (row >= p.M) continue;
      const int64_t srow = slot_row(row, pc.T, plan);
      const int64_t srow2 = slot_row(row, pc.T, plan2);
      const float a = am[b];
      const bool plain = a < 0x1p-100f || a > 0x1p+120f;
      const float y = 1.0f / a;
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t packed = 0u;
          if (a > 0.0f) {
            float qq[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float n = x[b][aa][4 * i + j] * QM;
              if (plain) {
                qq[j] = n / a;
              } else {
                qq[j] = n * y;
                const float r = __builtin_fmaf(-a, qq[j], n);
                qq[j] = __builtin_fmaf(r, y, qq[j]);
              }
            }
            if constexpr (EPI == 3) {
#pragma unroll
              for (int j = 0; j < 4; ++j)   // saturate overflowed quotients; keep the sign of zero
                qq[j] = __builtin_copysignf(fminf(fmaxf(qq[j], -448.0f), 448.0f), x[b][aa][4 * i + j]);
              packed = f32x2_to_e4m3x2(qq[0], qq[1], 0u, false);
              packed = f32x2_to_e4m3x2(qq[2], qq[3], packed, true);
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int qi = int(fminf(fmaxf(__builtin_rintf(qq[j]), -127.0f), 127.0f));
                packed |= (uint32_t(qi) & 0xffu) << (8 * j);
              }
            }
          }
          const int n_out = n0 + 64 * wn + 32 * aa + 8 * i + 4 * g;
          *reinterpret_cast<uint32_t*>(base + srow * N + n_out) = packed;
          if (srow2 >= 0) *reinterpret_cast<uint32_t*>(base + srow2 * N + n_out) = packed;
        }
      const int head = (n0 + 64 * wn) / pc.D;
      if (g == 0 && (pc.D == 64 || wn == 0)) {
        sc[srow * pc.H + head] = a / QM;
        if (srow2 >= 0) sc[srow2 * pc.H + head] = a / QM;
      }
    }
  }
}

// EPI 0: plain [M][N] outputs; 1: bf16 rows into cache slots; 2: int8 rows + scales;
// 3: fp8 (E4M3) rows + scales.
template <int EPI>
__global__ __launch_bounds__(NT, 2) void proj_kernel(const ProjToCacheParams pc, int n_mt, int n_units) {
  const ProjParams& p = pc.proj;
  __shared__ __attribute__((aligned(1024))) uint16_t sh0[TM * TK];
  __shared__ __attribute__((aligned(1024))) uint16_t sh1[TM * TK];
  __shared__ __attribute__((aligned(1024))) uint16_t sw0[TN * TK];
  __shared__ __attribute__((aligned(1024))) uint16_t sw1[TN * TK];

  // logical unit = (token tile, output tile, K/V); the units of one token tile are
  // consecutive and each XCD gets a contiguous range of units.
  const int per_xcd = (n_units + NXCD - 1) / NXCD;
  const int logical = (blockIdx.x % NXCD) * per_xcd + blockIdx.x / NXCD;
  if (logical >= n_units) return;
  const int n_nt = p.N / TN;
  const int mt = logical / (2 * n_nt);
  const int rem = logical % (2 * n_nt);
  const int nt = rem >> 1;
  const int z = rem & 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const int wm = wave & 1;     // token half
  const int wn = wave >> 1;    // output half
  const int m0 = mt * TM;
  const int n0 = nt * TN;
  const int m_valid = min(TM, p.M - m0);
  const uint16_t* W = z ? p.WV : p.WK;
  uint16_t* out = z ? p.outV : p.outK;

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  auto issue = [&](auto pb, int k0) __attribute__((always_inline)) {
    constexpr int PB = decltype(pb)::value;
    copy_tile<HCOPY>(p.h, p.K, m0, m_valid, k0, PB ? sh1 : sh0, wave, lane);
    copy_tile<WCOPY>(W, p.K, n0, TN, k0, PB ? sw1 : sw0, wave, lane);
  };
  auto compute = [&](auto pb) __attribute__((always_inline)) {
    constexpr int PB = decltype(pb)::value;
    const uint16_t* hs = PB ? sh1 : sh0;
    const uint16_t* ws = PB ? sw1 : sw0;
#pragma unroll
    for (int kk = 0; kk < TK / 16; ++kk) {
      bf16x8 af[2], bfr[4];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(ws + gswz(64 * wn + 32 * a + r32, 2 * kk + g)));
#pragma unroll
      for (int b = 0; b < 4; ++b)
        bfr[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(hs + gswz(128 * wm + 32 * b + r32, 2 * kk + g)));
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma32(af[a], bfr[b], acc[a][b]);
    }
  };
  auto step = [&](auto pb, int st, int nsteps) __attribute__((always_inline)) {
    constexpr int PB = decltype(pb)::value;
    if (st + 1 < nsteps) issue(std::integral_constant<int, PB ^ 1>{}, (st + 1) * TK);
    compute(pb);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  const int nsteps = p.K / TK;
  issue(std::integral_constant<int, 0>{}, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(std::integral_constant<int, 0>{}, st, nsteps);
    step(std::integral_constant<int, 1>{}, st + 1, nsteps);
  }
  if (st < nsteps) step(std::integral_constant<int, 0>{}, st, nsteps);

  // lane: token 128 wm + 32 b + r32, outputs 64 wn + 32 a + 8 i + 4 g + [0, 4)
  if constexpr (EPI == 0) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = m0 + 128 * wm + 32 * b + r32;
      if (row >= p.M) continue;
      uint16_t* dst = out + int64_t(row) * p.N + n0 + 64 * wn;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 w;
          w.x = pack_bf16x2(acc[a][b][4 * i + 0], acc[a][b][4 * i + 1]);
          w.y = pack_bf16x2(acc[a][b][4 * i + 2], acc[a][b][4 * i + 3]);
          *reinterpret_cast<u32x2*>(dst + 32 * a + 8 * i + 4 * g) = w;
        }
    }
  } else {
    cache_epilogue<EPI>(pc, acc, m0, n0, z, wm, wn, g, r32, tid);
  }
}

}  // namespace

namespace {
template <int EPI>
hipError_t launch_proj(const ProjToCacheParams& pc, hipStream_t s) {
  const ProjParams& p = pc.proj;
  if (p.K % TK != 0 || p.N % TN != 0 || p.M <= 0) return hipErrorInvalidValue;
  const int n_mt = (p.M + TM - 1) / TM;
  const int n_units = n_mt * (p.N / TN) * 2;
  const int grid = (n_units + NXCD - 1) / NXCD * NXCD;
  hipLaunchKernelGGL((proj_kernel<EPI>), dim3(grid), dim3(NT), 0, s, pc, n_mt, n_units);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_kv_project(const ProjParams& p, hipStream_t s) {
  ProjToCacheParams pc{};
  pc.proj = p;
  return launch_proj<0>(pc, s);
}

hipError_t launch_kv_project_to_cache(const ProjToCacheParams& p, hipStream_t s) {
  if (p.D != 64 && p.D != 128) return hipErrorInvalidValue;
  switch (p.kv_fmt) {
    case kKvBf16: return launch_proj<1>(p, s);
    case kKvInt8: return launch_proj<2>(p, s);
    case kKvFp8: return launch_proj<3>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ll
