// gemm.hip -- recache projection K_all = h W_K^T, V_all = h W_V^T (bf16 MFMA, fp32 sums).
//
// "LongLive: Real-time Interactive Long Video Generation" explainer, dpshk.com, §三
// item 4: self-attention keys and values are projections of the prompt-conditioned
// hidden state, K = W_K h', V = W_V h'; item 5: recache recomputes them for the
// retained latents under the new prompt.  W is the [d_out][d_in] matrix of that
// column form, so both operands are contiguous along the contraction d_in.
//
// Tiling: a workgroup of 4 waves computes 256 tokens x 128 outputs; each wave
// 128 tokens x 64 outputs with 32x32x16 bf16 MFMAs (W rows as the A operand, h rows
// as the B operand, so a lane's accumulators hold 4 consecutive outputs of one token
// and the bf16 results leave as 8-byte stores).  The contraction is walked in steps
// of 64 through double-buffered LDS fed by register prefetch.  blockIdx.z selects
// the K or the V projection, so both come from one launch.
#include "device_common.h"
#include "launch.h"

namespace ll {
namespace {

constexpr int TM = 256;     // tokens per workgroup
constexpr int TN = 128;     // outputs per workgroup
constexpr int TK = 64;      // contraction step
constexpr int PITCH = TK + 8;
constexpr int NT = 256;
constexpr int HPASS = TM * (TK / 8) / NT;   // 16-byte h chunks per thread per step (8)
constexpr int WPASS = TN * (TK / 8) / NT;   // 16-byte W chunks per thread per step (4)

__global__ __launch_bounds__(NT) void proj_kernel(const ProjParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sh[2][TM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sw[2][TN * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const int wm = wave & 1;     // token half
  const int wn = wave >> 1;    // output half
  const int m0 = blockIdx.x * TM;
  const int n0 = blockIdx.y * TN;
  const uint16_t* W = blockIdx.z ? p.WV : p.WK;
  uint16_t* out = blockIdx.z ? p.outV : p.outK;

  const int c = tid % 8;       // 16-byte chunk within a 64-element row
  const int rb = tid / 8;      // 0..31

  u32x4 ph[HPASS], pw[WPASS];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < HPASS; ++i) {
      const int row = m0 + rb + 32 * i;
      ph[i] = row < p.M ? *reinterpret_cast<const u32x4*>(p.h + int64_t(row) * p.K + k0 + 8 * c) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < WPASS; ++i) {
      const int row = n0 + rb + 32 * i;
      pw[i] = *reinterpret_cast<const u32x4*>(W + int64_t(row) * p.K + k0 + 8 * c);
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < HPASS; ++i) *reinterpret_cast<u32x4*>(&sh[b][(rb + 32 * i) * PITCH + 8 * c]) = ph[i];
#pragma unroll
    for (int i = 0; i < WPASS; ++i) *reinterpret_cast<u32x4*>(&sw[b][(rb + 32 * i) * PITCH + 8 * c]) = pw[i];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  const int nsteps = p.K / TK;
  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nsteps;
    if (more) load((st + 1) * TK);
    const uint16_t* hs = sh[buf];
    const uint16_t* ws = sw[buf];
#pragma unroll
    for (int kk = 0; kk < TK / 16; ++kk) {
      bf16x8 af[2], bfr[4];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(ws + (64 * wn + 32 * a + r32) * PITCH + 16 * kk + 8 * g));
#pragma unroll
      for (int b = 0; b < 4; ++b)
        bfr[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(hs + (128 * wm + 32 * b + r32) * PITCH + 16 * kk + 8 * g));
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma32(af[a], bfr[b], acc[a][b]);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
  }

  // lane: token 128 wm + 32 b + r32, outputs 64 wn + 32 a + 8 i + 4 g + [0, 4)
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
}

}  // namespace

hipError_t launch_kv_project(const ProjParams& p, hipStream_t s) {
  if (p.K % TK != 0 || p.N % TN != 0 || p.M <= 0) return hipErrorInvalidValue;
  dim3 grid(unsigned((p.M + TM - 1) / TM), unsigned(p.N / TN), 2);
  hipLaunchKernelGGL(proj_kernel, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace ll
