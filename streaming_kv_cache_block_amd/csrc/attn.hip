// attn.hip -- sink + window block-causal attention over the slot cache (gfx950).
//
// Computes, per head, softmax((Q K^T) / sqrt(D)) V of one chunk's queries over
//   segment 1: the cached slots [0, n_vis) (sink frames, then the window ring in
//              physical order -- "LongLive: Real-time Interactive Long Video
//              Generation" explainer, dpshk.com, §五 and §六: context = sink frames
//              plus the recent window);
//   segment 2: the chunk's own keys, all visible (block-causal mask, LongLive-2.0
//              explainer, wmrh.cn, §6: a chunk sees earlier chunks and itself).
// Nothing else is touched: evicted history is not in memory at all, and no mask is
// materialised -- the two segments ARE the visible set.
//
// Kernel structure (one workgroup = 4 waves, one head, 32*NQB query rows per wave):
//   * Q fragments stay in registers for the whole key walk.
//   * Keys are walked in tiles of 64 rows; each tile of K and V goes global ->
//     registers -> LDS (double-buffered, one barrier per tile) and is shared by
//     the 4 waves.  V is written to LDS transposed (V^T[d][key]) because the P*V
//     product contracts over keys; an XOR swizzle of 4-key quads keeps both the
//     transposed writes and the MFMA operand reads free of bank conflicts.
//   * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA:
//     each lane then holds one query's scores for 16 keys, so the running row max
//     needs one exchange with lane ^ 32 and the row sum is kept per lane (the two
//     halves are added once at the end).  The probabilities of the lane ARE the
//     MFMA B operand of O^T = V^T P^T: the keys of the lane's 8 B-slots are
//     matched by reading V^T at the same keys, so no register shuffle is needed.
//   * Online softmax in base 2 with log2(e)/sqrt(D) folded into one FMA.
//   * int8 caches: codes are widened to bf16 while staged into LDS (exact), the
//     per-key K scale multiplies the score column and the per-key V scale
//     multiplies the probability column before it is rounded to bf16
//     (LongLive-2.0 explainer, wmrh.cn, §15.3: dequantisation must not become a
//     separate slow pass).
#include "device_common.h"
#include "launch.h"

namespace ll {
namespace {

constexpr int BN = 64;        // keys per tile
constexpr int NTHREADS = 256; // 4 waves

template <int D>
struct Geo {
  static constexpr int KP = D + 8;          // K row pitch in LDS (elements): 16 B pad
  static constexpr int CH = D / 8;          // 8-element chunks per row
  static constexpr int KPASS = BN * CH / NTHREADS;  // 16-B K chunks per thread per tile
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int V_ELEMS = D * BN;    // V^T[d][key], 128 B rows, swizzled quads
};

// quad (4 keys = 8 bytes) position of key quad `q` in V^T row `d`
__device__ __forceinline__ int vt_quad(int d, int q) { return q ^ ((d ^ (d >> 3)) & 15); }

struct TileInfo {
  int seg;    // 0 = cache, 1 = own chunk
  int start;  // first key row of the tile within its segment
  int cnt;    // valid rows in the tile (1..BN)
};

__device__ __forceinline__ TileInfo tile_info(int j, int n1, int ncache, int nq) {
  TileInfo t;
  if (j < n1) {
    t.seg = 0;
    t.start = j * BN;
    t.cnt = min(BN, ncache - t.start);
  } else {
    t.seg = 1;
    t.start = (j - n1) * BN;
    t.cnt = min(BN, nq - t.start);
  }
  return t;
}

template <int D, bool KV8>
struct Stage {
  using G = Geo<D>;
  u32x4 k[G::KPASS];     // bf16 K chunks
  u32x4 v[4];            // bf16 V chunks: 4 keys x 8 d
  u32x2 k8[G::KPASS];    // int8 K chunks (cache tiles of int8 caches)
  u32x2 v8[4];
  float sc;              // K scale (threads 0..63) or V scale (64..127)
};

template <int D, bool KV8>
__device__ __forceinline__ void load_tile(Stage<D, KV8>& st, const AttnParams& p, const TileInfo& ti,
                                          int h, int tid) {
  using G = Geo<D>;
  const int64_t rs = int64_t(p.H) * D;   // row stride (elements)
  const int c = tid % G::CH;
  const bool int8_tile = KV8 && ti.seg == 0;
  // K: rows tid / CH + (NTHREADS / CH) * i
#pragma unroll
  for (int i = 0; i < G::KPASS; ++i) {
    const int r = tid / G::CH + (NTHREADS / G::CH) * i;
    const bool ok = r < ti.cnt;
    const int64_t off = int64_t(ti.start + r) * rs + int64_t(h) * D + 8 * c;
    if (int8_tile) {
      st.k8[i] = ok ? *reinterpret_cast<const u32x2*>(static_cast<const int8_t*>(p.cK) + off) : u32x2{0, 0};
    } else {
      const uint16_t* base = ti.seg == 0 ? static_cast<const uint16_t*>(p.cK) : p.Kc;
      st.k[i] = ok ? *reinterpret_cast<const u32x4*>(base + off) : u32x4{0, 0, 0, 0};
    }
  }
  // V: 4 consecutive keys 4*kq .. 4*kq+3, chunk c
  const int kq = tid / G::CH;
  if (kq < BN / 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * kq + i;
      const bool ok = r < ti.cnt;
      const int64_t off = int64_t(ti.start + r) * rs + int64_t(h) * D + 8 * c;
      if (int8_tile) {
        st.v8[i] = ok ? *reinterpret_cast<const u32x2*>(static_cast<const int8_t*>(p.cV) + off) : u32x2{0, 0};
      } else {
        const uint16_t* base = ti.seg == 0 ? static_cast<const uint16_t*>(p.cV) : p.Vc;
        st.v[i] = ok ? *reinterpret_cast<const u32x4*>(base + off) : u32x4{0, 0, 0, 0};
      }
    }
  }
  if (KV8) {
    st.sc = 1.0f;
    if (int8_tile && tid < 2 * BN) {
      const int r = tid % BN;
      const float* sp = tid < BN ? p.cKs : p.cVs;
      st.sc = r < ti.cnt ? sp[int64_t(ti.start + r) * p.H + h] : 0.0f;
    }
  }
}

template <int D, bool KV8>
__device__ __forceinline__ void store_tile(const Stage<D, KV8>& st, uint16_t* ks, uint16_t* vt, float* kscl,
                                           float* vscl, const TileInfo& ti, int tid) {
  using G = Geo<D>;
  const int c = tid % G::CH;
  const bool int8_tile = KV8 && ti.seg == 0;
#pragma unroll
  for (int i = 0; i < G::KPASS; ++i) {
    const int r = tid / G::CH + (NTHREADS / G::CH) * i;
    u32x4 w;
    if (int8_tile) {
      w = u32x4{i8x2_to_bf16x2(st.k8[i].x, 0), i8x2_to_bf16x2(st.k8[i].x, 2),
                i8x2_to_bf16x2(st.k8[i].y, 0), i8x2_to_bf16x2(st.k8[i].y, 2)};
    } else {
      w = st.k[i];
    }
    *reinterpret_cast<u32x4*>(ks + r * G::KP + 8 * c) = w;
  }
  const int kq = tid / G::CH;
  if (kq < BN / 4) {
    u32x4 rv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (int8_tile) {
        rv[i] = u32x4{i8x2_to_bf16x2(st.v8[i].x, 0), i8x2_to_bf16x2(st.v8[i].x, 2),
                      i8x2_to_bf16x2(st.v8[i].y, 0), i8x2_to_bf16x2(st.v8[i].y, 2)};
      } else {
        rv[i] = st.v[i];
      }
    }
    // rv[i] holds V[4kq+i][8c .. 8c+7]; write V^T[8c+j][4kq .. 4kq+3] for j < 8
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = 8 * c + j;
      const int w = j >> 1;
      u32x2 q;
      if (j & 1) {
        q.x = pick_hi_hi(rv[0][w], rv[1][w]);
        q.y = pick_hi_hi(rv[2][w], rv[3][w]);
      } else {
        q.x = pick_lo_lo(rv[0][w], rv[1][w]);
        q.y = pick_lo_lo(rv[2][w], rv[3][w]);
      }
      *reinterpret_cast<u32x2*>(vt + d * BN + 4 * vt_quad(d, kq)) = q;
    }
  }
  if (KV8 && tid < 2 * BN) {
    (tid < BN ? kscl : vscl)[tid % BN] = st.sc;
  }
}

template <int D, int NQB, bool KV8>
__global__ __launch_bounds__(NTHREADS) void attn_kernel(const AttnParams p) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sm_k[2][G::K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sm_v[2][G::V_ELEMS];
  __shared__ __attribute__((aligned(16))) float sm_ks[KV8 ? 2 : 1][BN];
  __shared__ __attribute__((aligned(16))) float sm_vs[KV8 ? 2 : 1][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;     // lane half
  const int r32 = lane & 31;
  const int h = blockIdx.y;
  const int64_t rs = int64_t(p.H) * D;
  const int q0 = blockIdx.x * (4 * 32 * NQB) + wave * (32 * NQB);

  // Q^T fragments (MFMA B operand): lane holds query r32, d = 16 s + 8 g + [0, 8)
  bf16x8 qf[NQB][D / 16];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = q0 + 32 * qb + r32;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 w = {0, 0, 0, 0};
      if (row < p.nq) w = *reinterpret_cast<const u32x4*>(p.Q + int64_t(row) * rs + int64_t(h) * D + 16 * s + 8 * g);
      qf[qb][s] = as_bf16x8(w);
    }
  }

  f32x16 O[NQB][D / 32];
  float m[NQB], l[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = -__builtin_inff();
    l[qb] = 0.0f;
#pragma unroll
    for (int e = 0; e < D / 32; ++e) O[qb][e] = f32x16{};
  }

  const int n1 = (p.ncache + BN - 1) / BN;
  const int ntiles = n1 + (p.nq + BN - 1) / BN;
  const float c = p.c;

  Stage<D, KV8> st;
  TileInfo ti = tile_info(0, n1, p.ncache, p.nq);
  load_tile<D, KV8>(st, p, ti, h, tid);
  store_tile<D, KV8>(st, sm_k[0], sm_v[0], sm_ks[0], sm_vs[0], ti, tid);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const TileInfo cur = ti;
    const bool more = j + 1 < ntiles;
    if (more) {
      ti = tile_info(j + 1, n1, p.ncache, p.nq);
      load_tile<D, KV8>(st, p, ti, h, tid);
    }
    const uint16_t* ks = sm_k[buf];
    const uint16_t* vt = sm_v[buf];

    // ---- S^T = K Q^T for 64 keys (two 32-key blocks) ----
    f32x16 S[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) S[qb][0] = S[qb][1] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 k0 = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + r32 * G::KP + 16 * s + 8 * g));
      const bf16x8 k1 = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + (32 + r32) * G::KP + 16 * s + 8 * g));
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        S[qb][0] = mfma32(k0, qf[qb][s], S[qb][0]);
        S[qb][1] = mfma32(k1, qf[qb][s], S[qb][1]);
      }
    }

    const bool scaled = KV8 && cur.seg == 0;
    if (scaled) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 kscv = *reinterpret_cast<const f32x4*>(&sm_ks[KV8 ? buf : 0][32 * b + 8 * i + 4 * g]);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[qb][b][4 * i + jj] *= kscv[jj];
        }
    }
    if (cur.cnt < BN) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int key = 32 * b + 8 * i + 4 * g + jj;
            if (key >= cur.cnt) {
#pragma unroll
              for (int qb = 0; qb < NQB; ++qb) S[qb][b][4 * i + jj] = -__builtin_inff();
            }
          }
    }

    // ---- online softmax (base 2) ----
    bf16x8 P[NQB][4];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = S[qb][0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[qb][b][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[qb], mx * c);
      const float alpha = fast_exp2(m[qb] - mnew);
      m[qb] = mnew;
      float rsum = 0.0f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = fast_exp2(__builtin_fmaf(S[qb][b][v], c, -mnew));
          rsum += e;
          S[qb][b][v] = e;
        }
      l[qb] = l[qb] * alpha + rsum;
#pragma unroll
      for (int e = 0; e < D / 32; ++e) O[qb][e] *= alpha;
      if (scaled) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 vscv = *reinterpret_cast<const f32x4*>(&sm_vs[KV8 ? buf : 0][32 * b + 8 * i + 4 * g]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[qb][b][4 * i + jj] *= vscv[jj];
          }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = u >> 1, v0 = 8 * (u & 1);
        u32x4 w;
        w.x = pack_bf16x2(S[qb][b][v0 + 0], S[qb][b][v0 + 1]);
        w.y = pack_bf16x2(S[qb][b][v0 + 2], S[qb][b][v0 + 3]);
        w.z = pack_bf16x2(S[qb][b][v0 + 4], S[qb][b][v0 + 5]);
        w.w = pack_bf16x2(S[qb][b][v0 + 6], S[qb][b][v0 + 7]);
        P[qb][u] = as_bf16x8(w);
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int e = 0; e < D / 32; ++e) {
      const int d = 32 * e + r32;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int qd1 = 8 * (u >> 1) + 4 * (u & 1) + g;   // quad of keys 32b + 16(u&1) + 4g
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vt + d * BN + 4 * vt_quad(d, qd1));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vt + d * BN + 4 * vt_quad(d, qd1 + 2));
        const bf16x8 vf = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) O[qb][e] = mfma32(vf, P[qb][u], O[qb][e]);
      }
    }

    if (more) {
      const int nb = buf ^ 1;
      store_tile<D, KV8>(st, sm_k[nb], sm_v[nb], sm_ks[KV8 ? nb : 0], sm_vs[KV8 ? nb : 0], ti, tid);
    }
    __syncthreads();
  }

  // ---- normalise and store O (lane: query r32, d = 32 e + 8 i + 4 g + [0, 4)) ----
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const float inv = 1.0f / lt;
    const int row = q0 + 32 * qb + r32;
    if (row < p.nq) {
      uint16_t* dst = p.out + int64_t(row) * rs + int64_t(h) * D;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 w;
          w.x = pack_bf16x2(O[qb][e][4 * i + 0] * inv, O[qb][e][4 * i + 1] * inv);
          w.y = pack_bf16x2(O[qb][e][4 * i + 2] * inv, O[qb][e][4 * i + 3] * inv);
          *reinterpret_cast<u32x2*>(dst + 32 * e + 8 * i + 4 * g) = w;
        }
    }
  }
}

template <int D, int NQB, bool KV8>
hipError_t launch_t(const AttnParams& p, hipStream_t s) {
  const int rows = 4 * 32 * NQB;
  dim3 grid((p.nq + rows - 1) / rows, p.H);
  hipLaunchKernelGGL((attn_kernel<D, NQB, KV8>), grid, dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int D, bool kv_int8, hipStream_t s) {
  const bool big = p.nq > 4 * 32;
  if (D == 128) {
    // one 32-row block per wave: two blocks per wave exceed the register file
    if (kv_int8) return launch_t<128, 1, true>(p, s);
    return launch_t<128, 1, false>(p, s);
  }
  if (D == 64) {
    if (kv_int8) return big ? launch_t<64, 2, true>(p, s) : launch_t<64, 1, true>(p, s);
    return big ? launch_t<64, 2, false>(p, s) : launch_t<64, 1, false>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ll
