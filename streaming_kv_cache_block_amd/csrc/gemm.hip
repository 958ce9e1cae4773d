// gemm.hip -- recache projection K_all = h W_K^T, V_all = h W_V^T (bf16 MFMA, fp32 sums).
//
// "LongLive: Real-time Interactive Long Video Generation" explainer, dpshk.com, §三
// item 4: self-attention keys and values are projections of the prompt-conditioned
// hidden state, K = W_K h', V = W_V h'; item 5: recache recomputes them for the
// retained latents under the new prompt.  W is the [d_out][d_in] matrix of that
// column form, so both operands are contiguous along the contraction d_in.
//
// Tiling: a workgroup computes TM tokens x TN outputs with 2 TN / 64 waves, each TM / 2
// tokens x 64 outputs with 32x32x16 bf16 MFMAs (W rows as the A operand, h rows as the
// B operand, so a lane's accumulators hold 4 consecutive outputs of one token and the
// bf16 results leave as 8-byte stores).  The contraction is walked in steps of TK: each
// step's h and W tiles are copied global -> LDS with the buffer load-to-LDS path
// (buffer_load ... lds; the global form would make the compiler wait for every LDS read
// in flight before each MFMA, see the attention kernel's copy_lds) into two
// buffers that are separate LDS objects (buffer parity fixed at compile time, so the
// copy of step s+1 overlaps the MFMAs of step s).  The 16-byte chunks of a row are
// XOR-swizzled so that the 16 rows one operand read touches land on 16 distinct bank
// groups.  Tile shapes are listed at Shape below.  Each unit is one (token tile, output
// tile, K or V) triple; workgroups that share an h tile run on the same XCD.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ll {
namespace {

constexpr int NXCD = 8;

// Tile shapes: TM tokens x TN outputs per workgroup of 2 TN / 64 waves, each TM / 2
// tokens x 64 outputs, contraction steps of TK, MINB workgroups per CU.  The larger the
// tile, the more multiply-adds each byte copied global -> LDS feeds, which is what
// bounds this kernel: 192 x 384 with TK = 64 (12 waves, three per SIMD, 144 KB of
// double-buffered LDS) for output counts that are a multiple of 384, 192 x 256 (8
// waves, 112 KB) for other multiples of 256, 256 x 128 with TK = 32 (4 waves, two
// workgroups per CU) for the rest.
template <int TM_, int TN_, int TK_, int MINB_>
struct Shape {
  static constexpr int TM = TM_, TN = TN_, TK = TK_, MINB = MINB_;
  static constexpr int MB = TM / 64;                 // 32-token blocks per wave
  static constexpr int WM = TM / 2;                  // tokens per wave
  static constexpr int NW = 2 * TN / 64;             // waves
  static constexpr int NT = 64 * NW;                 // threads
  static constexpr int HCOPY = TM * TK * 2 / 1024;   // 1 KB wave-wide copies of the h tile
  static constexpr int WCOPY = TN * TK * 2 / 1024;   // of the W tile
  static constexpr int CPR = TK / 8;                 // 16-byte chunks per row
  static constexpr int RPC = 64 / CPR;               // rows per wave-wide copy
  static_assert(HCOPY % NW == 0 && WCOPY % NW == 0, "copies per wave");
};

typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzle of row r: the 16 rows one operand read serves together land on 16
// distinct 16-byte bank groups (64-byte rows: r >> 2; 128-byte rows: r >> 1, the row
// parity already splits the 256-byte bank window).
template <int TK>
__device__ __forceinline__ int swz_of(int r) {
  if constexpr (TK == 32) return (r >> 2) & 3;
  else return (r >> 1) & 7;
}
// element offset of 16-byte chunk c of row r in a swizzled [rows][TK] tile
template <int TK>
__device__ __forceinline__ int gswz(int r, int c) { return r * TK + 8 * (c ^ swz_of<TK>(r)); }

// Copy rows [0, rows) x [k0, k0 + TK) of a row-major [*, ld] bf16 matrix into LDS.
// Lane l of copy i fills LDS bytes [1 KB i + 16 l, +16): row RPC i + l / CPR, chunk
// position l % CPR, which holds source chunk (l % CPR) ^ swz(row).
template <class SH, int NCOPY>
__device__ __forceinline__ void copy_tile(const uint16_t* g, int64_t ld, int row0, int rows_valid, int k0,
                                          uint16_t* lds, int wave, int lane) {
  constexpr int TK = SH::TK;
  const uint16_t* base = g + int64_t(row0) * ld + k0;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, int(rows_valid * ld * 2), 0x00020000);
#pragma unroll
  for (int i = wave; i < NCOPY; i += SH::NW) {
    const int r = SH::RPC * i + lane / SH::CPR;
    const int c = (lane % SH::CPR) ^ swz_of<TK>(r);
    const int rr = min(r, rows_valid - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + SH::RPC * i * TK), 16,
                                             int(rr * ld + 8 * c) * 2, 0, 0, 0);
  }
}

// Row of the cache slot array that output row m lands in: frame m / T goes to slot
// plan[m / T] (plan in LDS), token m % T; -1 when the plan has no slot there.
__device__ __forceinline__ int64_t slot_row(int m, int T, const int* plan) {
  const int s = plan[m / T];
  return s < 0 ? -1 : int64_t(s) * T + m % T;
}

// Epilogue of the fused recache: bf16 results, their MX quantisation (below), or their
// int8 / fp8 quantisation
//   a = max |x| over the (token, head) row, scale = a / M,
//   q = clamp(rint((x * M) / a), -M, M) with M = 127   (0 for an all-zero row),
//   or the E4M3 rounding of clamp((x * M) / a, -M, M) with M = 448,
// with the quotient correctly rounded as in the int8 cache writer (one IEEE reciprocal
// per row and a Markstein FMA correction; plain division where the absmax is below
// 2^-100 or above 2^120).  x is the bf16-rounded sum, exactly what a separate
// projection would have stored.
template <int EPI, class SH>
__device__ __forceinline__ void cache_epilogue(const ProjToCacheParams& pc, const f32x16 (&acc)[2][SH::MB], int m0,
                                               int n0, int z, int wm, int wn, int g, int r32, int tid) {
  constexpr int MB = SH::MB, WM = SH::WM, TN = SH::TN;
  // A frame may be held by two slots (a shot-sink frame still in the window): the row
  // is then written to both.
  __shared__ int plan[kMaxPlan], plan2[kMaxPlan];
  __shared__ float amax[2][TN / 64][WM];   // [wm][wn][token within the wave's half]
  const ProjParams& p = pc.proj;
  for (int i = tid; i < pc.n_plan; i += SH::NT) {
    plan[i] = pc.plan_slot[i];
    plan2[i] = pc.plan_slot2[i];
  }
  __syncthreads();
  const int N = p.N;
  if constexpr (EPI == 1) {
    uint16_t* base = static_cast<uint16_t*>(z ? pc.slotV : pc.slotK);
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int row = m0 + WM * wm + 32 * b + r32;
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
  } else if constexpr (EPI >= 4) {
    // MX caches (4: MXFP4, E2M1 codes; 5: MXFP8, E4M3 codes), one power-of-two scale per
    // block of 32 values, the rule of the MX cache writer: a block is half a wave's 64
    // outputs (32 a ..), held by the lane pair (g = 0, 1) of a token, so its absmax takes
    // one exchange; e = max(floor(log2 a) - EMAX, EMIN) from the bf16 absmax's exponent
    // field, y = x * 2^-e (exact), the hardware conversion with unit scale (E4M3 values
    // clamped to +-448 first).  A wave's 64 outputs are one head (D = 64, blocks 0, 1) or
    // half of one (D = 128, blocks 0, 1 or 2, 3): its two scale bytes go out in one store.
    constexpr bool FP4 = EPI == 4;
    constexpr int EMAX = FP4 ? 2 : 8;
    constexpr int EMIN = FP4 ? -125 : -117;
    float x[MB][2][16];
    int eb[MB][2];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float mx = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          x[b][a][v] = __builtin_bit_cast(float, pack_bf16x2(acc[a][b][v], 0.0f) << 16);
          mx = fmaxf(mx, fabsf(x[b][a][v]));
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        eb[b][a] = max(int(__builtin_bit_cast(uint32_t, mx) >> 23) - 127 - EMAX, EMIN);
      }
    uint8_t* base = static_cast<uint8_t*>(z ? pc.slotV : pc.slotK);
    uint8_t* scb = reinterpret_cast<uint8_t*>(z ? pc.scV : pc.scK);
    const int head = (n0 + 64 * wn) / pc.D;
    const int blk0 = ((n0 + 64 * wn) % pc.D) / 32;   // the head's block of half a = 0
    const int64_t rb = FP4 ? N / 2 : N;              // code bytes per token row
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int row = m0 + WM * wm + 32 * b + r32;
      if (row >= p.M) continue;
      const int64_t srow = slot_row(row, pc.T, plan);
      const int64_t srow2 = slot_row(row, pc.T, plan2);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const float inv = __builtin_bit_cast(float, uint32_t(127 - eb[b][a]) << 23);   // 2^-e
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* xv = &x[b][a][4 * i];
          const int n_out = n0 + 64 * wn + 32 * a + 8 * i + 4 * g;
          if constexpr (FP4) {
            uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, xv[0] * inv, xv[1] * inv, 1.0f, 0);
            c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, xv[2] * inv, xv[3] * inv, 1.0f, 1);
            *reinterpret_cast<uint16_t*>(base + srow * rb + n_out / 2) = uint16_t(c);
            if (srow2 >= 0) *reinterpret_cast<uint16_t*>(base + srow2 * rb + n_out / 2) = uint16_t(c);
          } else {
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = fminf(fmaxf(xv[j] * inv, -448.0f), 448.0f);
            uint32_t c = f32x2_to_e4m3x2(y[0], y[1], 0u, false);
            c = f32x2_to_e4m3x2(y[2], y[3], c, true);
            *reinterpret_cast<uint32_t*>(base + srow * rb + n_out) = c;
            if (srow2 >= 0) *reinterpret_cast<uint32_t*>(base + srow2 * rb + n_out) = c;
          }
        }
      }
      if (g == 0) {
        const uint32_t two = uint32_t(eb[b][0] + 127) | (uint32_t(eb[b][1] + 127) << 8);
        for (int k = 0; k < 2; ++k) {
          const int64_t sr = k ? srow2 : srow;
          if (sr < 0) continue;
          uint8_t* w = scb + (sr * pc.H + head) * 4;
          if (pc.D == 64) *reinterpret_cast<uint32_t*>(w) = two;   // bytes 2, 3 stay 0
          else *reinterpret_cast<uint16_t*>(w + blk0) = uint16_t(two);
        }
      }
    }
  } else {
    // bf16-round, then the absmax of each (token, head) row: 32 values per lane, lanes
    // g = 0/1 hold a wave's 64 outputs; with D = 128 the two waves of a head (wn, wn ^ 1)
    // combine through LDS, with D = 64 a wave's 64 outputs are one head.
    float x[MB][2][16];
    float am[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
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
        for (int b = 0; b < MB; ++b) amax[wm][wn][32 * b + r32] = am[b];
      }
      __syncthreads();
#pragma unroll
      for (int b = 0; b < MB; ++b) am[b] = fmaxf(am[b], amax[wm][wn ^ 1][32 * b + r32]);
    }
    constexpr float QM = EPI == 3 ? 448.0f : 127.0f;
    int8_t* base = static_cast<int8_t*>(z ? pc.slotV : pc.slotK);
    float* sc = z ? pc.scV : pc.scK;
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int row = m0 + WM * wm + 32 * b + r32;
      if (row >= p.M) continue;
      const int64_t srow = slot_row(row, pc.T, plan);
      const int64_t srow2 = slot_row(row, pc.T, plan2);
      const float a = am[b];
      const bool plain = a < 0x1p-100f || a > 0x1p+120f;
      const float y = 1.0f / a;
      // codes of values 4 i .. 4 i + 3 of half aa; GEN: any row of the wave may be zero
      // or outside [2^-100, 2^120] (plain division), else the Markstein path only
      auto q4 = [&](auto general, int aa, int i) __attribute__((always_inline)) -> uint32_t {
        constexpr bool GEN = decltype(general)::value;
        uint32_t packed = 0u;
        if (!GEN || a > 0.0f) {
          float qq[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float n = x[b][aa][4 * i + j] * QM;
            if (GEN && plain) {
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
        return packed;
      };
      // the test is made once per wave, so that the common case has no branch per value
      uint32_t pk[2][4];
      if (__builtin_amdgcn_ballot_w64(plain || !(a > 0.0f)) == 0) {
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[aa][i] = q4(std::false_type{}, aa, i);
      } else {
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[aa][i] = q4(std::true_type{}, aa, i);
      }
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n_out = n0 + 64 * wn + 32 * aa + 8 * i + 4 * g;
          *reinterpret_cast<uint32_t*>(base + srow * N + n_out) = pk[aa][i];
          if (srow2 >= 0) *reinterpret_cast<uint32_t*>(base + srow2 * N + n_out) = pk[aa][i];
        }
      const int head = (n0 + 64 * wn) / pc.D;
      if (g == 0 && (pc.D == 64 || (wn & 1) == 0)) {
        sc[srow * pc.H + head] = a / QM;
        if (srow2 >= 0) sc[srow2 * pc.H + head] = a / QM;
      }
    }
  }
}

// EPI 0: plain [M][N] outputs; 1: bf16 rows into cache slots; 2: int8 rows + scales;
// 3: fp8 (E4M3) rows + scales; 4: MXFP4 rows + block scales; 5: MXFP8 rows + block scales.
template <int EPI, class SH>
__global__ __launch_bounds__(SH::NT, SH::MINB) void proj_kernel(const ProjToCacheParams pc, int n_mt, int n_units) {
  constexpr int TM = SH::TM, TN = SH::TN, TK = SH::TK;
  constexpr int MB = SH::MB, WM = SH::WM;
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const int wm = wave & 1;     // token half
  const int wn = wave >> 1;    // 64-output part
  const int m0 = mt * TM;
  const int n0 = nt * TN;
  const int m_valid = min(TM, p.M - m0);
  const uint16_t* W = z ? p.WV : p.WK;
  uint16_t* out = z ? p.outV : p.outK;

  f32x16 acc[2][MB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[a][b] = f32x16{};

  auto issue = [&](auto pb, int k0) __attribute__((always_inline)) {
    constexpr int PB = decltype(pb)::value;
    copy_tile<SH, SH::HCOPY>(p.h, p.K, m0, m_valid, k0, PB ? sh1 : sh0, wave, lane);
    copy_tile<SH, SH::WCOPY>(W, p.K, n0, TN, k0, PB ? sw1 : sw0, wave, lane);
  };
  auto compute = [&](auto pb) __attribute__((always_inline)) {
    constexpr int PB = decltype(pb)::value;
    const uint16_t* hs = PB ? sh1 : sh0;
    const uint16_t* ws = PB ? sw1 : sw0;
#pragma unroll
    for (int kk = 0; kk < TK / 16; ++kk) {
      bf16x8 af[2], bfr[MB];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(ws + gswz<TK>(64 * wn + 32 * a + r32, 2 * kk + g)));
#pragma unroll
      for (int b = 0; b < MB; ++b)
        bfr[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(hs + gswz<TK>(WM * wm + 32 * b + r32, 2 * kk + g)));
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = mfma32(af[a], bfr[b], acc[a][b]);
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
    for (int b = 0; b < MB; ++b) {
      const int row = m0 + WM * wm + 32 * b + r32;
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
    cache_epilogue<EPI, SH>(pc, acc, m0, n0, z, wm, wn, g, r32, tid);
  }
}

}  // namespace

namespace {
template <int EPI, class SH>
hipError_t launch_shape(const ProjToCacheParams& pc, hipStream_t s) {
  const ProjParams& p = pc.proj;
  const int n_mt = (p.M + SH::TM - 1) / SH::TM;
  const int n_units = n_mt * (p.N / SH::TN) * 2;
  const int grid = (n_units + NXCD - 1) / NXCD * NXCD;
  hipLaunchKernelGGL((proj_kernel<EPI, SH>), dim3(grid), dim3(SH::NT), 0, s, pc, n_mt, n_units);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_proj(const ProjToCacheParams& pc, hipStream_t s) {
  const ProjParams& p = pc.proj;
  if (p.K % 64 != 0 || p.N % 128 != 0 || p.M <= 0) return hipErrorInvalidValue;
  // 192 x 384 tiles at the recache size (23400 tokens x 2 x 1536 outputs): 122 x 8
  // units fill 256 CUs in 3.8 rounds, and each copied byte feeds 64 multiply-adds
  // (55 for 192 x 256; 256-token tiles would leave most of the chip idle in the last
  // round).
  if (p.N % 384 == 0) return launch_shape<EPI, Shape<192, 384, 64, 1>>(pc, s);
  if (p.N % 256 == 0) return launch_shape<EPI, Shape<192, 256, 64, 1>>(pc, s);
  return launch_shape<EPI, Shape<256, 128, 32, 2>>(pc, s);
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
    case kKvMxfp4: return launch_proj<4>(p, s);
    case kKvMxfp8: return launch_proj<5>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ll
