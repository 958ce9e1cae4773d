// attn.hip -- sink + window block-causal attention over the slot cache (gfx950).
//
// Computes, per head, softmax((Q K^T) / sqrt(D)) V of one chunk's queries over
//   segment 1: the cached slots [0, n_vis) (sink frames, then the window ring in
//              physical order -- "LongLive: Real-time Interactive Long Video
//              Generation" explainer, dpshk.com, §五 and §六: the context is the
//              sink frames plus the recent window);
//   segment 2: the chunk's own keys, all visible (block-causal mask, LongLive-2.0
//              explainer, wmrh.cn, §6: a chunk sees earlier chunks and itself).
// Evicted history is not in memory and no mask is materialised: the two segments
// are the visible set, walked in tiles of 64 keys; only a segment's last tile is
// partial.
//
// Workgroup = NW waves, one head, 32*NQB query rows per wave (NQB 32-row blocks).
//   * Q fragments stay in registers for the whole key walk.
//   * K and V tiles live in LDS in their natural [key][d] layout, double-buffered,
//     one barrier per tile.  16-byte chunks are XOR-swizzled per row so that the
//     MFMA operand reads below are free of bank conflicts.  bf16 tiles are copied
//     global -> LDS by the buffer load-to-LDS path (no registers); int8 / fp8 cache
//     tiles are copied as codes into a per-wave staging area the same way and widened
//     to bf16 by that wave (exact: |q| <= 127, and every E4M3 value is a bf16 value).
//   * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA: a
//     lane then holds one query's scores for 16 keys of each 32-key block, so the
//     running row max needs one register exchange with lane ^ 32
//     (v_permlane32_swap) and the row sum stays per lane until the end.  Each K
//     fragment read from LDS feeds NQB MFMAs.
//   * The lane's probabilities are the B operand of O^T = V^T P^T as they are; the
//     A operand V^T (8 keys of one d per lane, keys matched to the lane's B slots)
//     comes from two transpose reads (ds_read_b64_tr_b16) of the natural V tile.
//   * Online softmax in base 2, log2(e)/sqrt(D) folded into one FMA; the running
//     max is only raised (and O, l rescaled) when a score exceeds it by more than
//     2^8, which keeps every probability <= 256 and skips almost all rescales.
//     Full bf16 tiles first take the probabilities against the running max as it
//     stands and check the bound on the lane's tile sum; only tiles that fail it
//     (rare after the first) compute the tile max, rescale and take them again.
//   * int8 / fp8 caches: the per-key K scale multiplies the score column and the V
//     scale the probability column before rounding to bf16 (LongLive-2.0 explainer,
//     wmrh.cn, §15.3: dequantisation fused into the consumer, not a separate pass).
//   * Workgroups are numbered so that the query tiles of one head run on the same
//     XCD (consecutive workgroup ids are dealt round-robin to the 8 XCDs) and share
//     its L2 while they stream the same keys.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ll {
namespace {

constexpr int BN = 64;         // keys per tile
constexpr int NXCD = 8;
constexpr float kLazyThreshold = 8.0f;   // log2 units
#ifndef LL_PIECE_TILES
#define LL_PIECE_TILES 12
#endif
constexpr int kPieceTiles = LL_PIECE_TILES;   // per-piece overhead of a split walk, in tiles
#ifndef LL_SPEC
#define LL_SPEC 1
#endif
constexpr bool kSpecSoftmax = LL_SPEC;   // full bf16 tiles: probabilities against the running max first

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

template <int D, int NW>
struct Geo {
  static constexpr int NT = 64 * NW;                   // threads per workgroup
  static constexpr int CH = D / 8;                     // 16-byte chunks per row
  static constexpr int ROWS_PER_DMA = 64 / CH;         // rows one wave-wide 1 KB copy covers
  static constexpr int DMA_PER_WAVE = BN / ROWS_PER_DMA / NW;
  static constexpr int REG_PASS = BN * CH / NT;        // int8 staging: chunks per thread
  static constexpr int TILE = BN * D;                  // elements per K (or V) tile
  static_assert(DMA_PER_WAVE >= 1 && REG_PASS >= 1 && NT >= 2 * BN, "tile split");
};

// Swizzled chunk position of chunk c in row r.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  else return c ^ (((r & 1) << 2) | ((r >> 1) & 3));
}

// Element offset of chunk c of row r in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz_row_base(int r, int c) {
  return r * D + 8 * swz<D>(r, c);
}

// One wave-wide copy global -> LDS of BYTES per lane (lane l lands at lds + BYTES l)
// from the wave-uniform base plus the lane's byte offset voff, in the buffer form
// (buffer_load ... lds; the offset range check is left open).  Not the global form:
// the compiler counts a pending global-form load-to-LDS as an access to both memory
// and LDS, and then makes every LDS read after it wait for all LDS reads in flight
// (lgkmcnt(0)), which serialises the operand reads with the MFMAs that consume them.
template <int BYTES>
__device__ __forceinline__ void copy_lds(const void* base, uint32_t voff, void* lds) {
  static_assert(BYTES == 16 || BYTES == 4, "copy width");
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
  if constexpr (BYTES == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, int(voff), 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, int(voff), 0, 0, 0);
}

struct TileInfo {
  int seg;    // 0 = cache, 1 = own chunk
  int start;  // first key row of the tile within its segment
  int cnt;    // valid rows in the tile (1..BN)
};

// bf16 tile: every wave copies its share of rows straight into LDS.  Rows past the
// segment end re-read the last valid row (its scores are masked to -inf and its
// values then get probability 0, so the data only has to be finite).
template <int D, int NW>
__device__ __forceinline__ void dma_tile(const uint16_t* gk, const uint16_t* gv, int64_t rs, const TileInfo& ti,
                                         uint16_t* lk, uint16_t* lv, int wave, int lane) {
  using G = Geo<D, NW>;
#pragma unroll
  for (int i = 0; i < G::DMA_PER_WAVE; ++i) {
    const int r0 = (wave * G::DMA_PER_WAVE + i) * G::ROWS_PER_DMA;
    const int r = r0 + lane / G::CH;
    const int c = swz<D>(r, lane % G::CH);
    const int64_t base = int64_t(ti.start) * rs;
    const uint32_t off = uint32_t((int64_t(min(r, ti.cnt - 1)) * rs + 8 * c) * 2);
    copy_lds<16>(gk + base, off, lk + r0 * D);
    copy_lds<16>(gv + base, off, lv + r0 * D);
  }
}

// Full bf16 tile: the per-lane byte offsets of the rows and chunks a wave copies are
// the same for every tile (loff, computed once); the tile start only moves the
// wave-uniform base pointers gk/gv.
template <int D, int NW>
__device__ __forceinline__ void dma_full(const uint16_t* gk, const uint16_t* gv, const uint32_t* loff,
                                         uint16_t* lk, uint16_t* lv, int wave) {
  using G = Geo<D, NW>;
#pragma unroll
  for (int i = 0; i < G::DMA_PER_WAVE; ++i) {
    const int r0 = (wave * G::DMA_PER_WAVE + i) * G::ROWS_PER_DMA;
    copy_lds<16>(gk, loff[i], lk + r0 * D);
    copy_lds<16>(gv, loff[i], lv + r0 * D);
  }
}

template <int D, int NW>
__device__ __forceinline__ uint32_t dma_lane_offset(int64_t rs, int wave, int lane, int i) {
  using G = Geo<D, NW>;
  const int r = (wave * G::DMA_PER_WAVE + i) * G::ROWS_PER_DMA + lane / G::CH;
  return uint32_t((int64_t(r) * rs + 8 * swz<D>(r, lane % G::CH)) * 2);
}

// Quantised cache tile (int8 or fp8 codes): each wave copies whole rows of raw codes
// into a staging area (load-to-LDS, natural [row][D bytes] layout) and, after its own
// copies have landed, widens exactly those rows to bf16 in the swizzled tile buffer
// (exact: |q| <= 127, and every E4M3 value is a bf16 value).
// No wave reads another wave's staging rows, so no barrier is needed in between.  The
// per-row scales are copied straight into their LDS arrays by waves 0 (K) and 1 (V).
template <int D, int NW, int FMT>
struct QTile {
  static constexpr int CH8 = D / 16;                 // 16-byte chunks per int8 row
  static constexpr int ROWS = 64 / CH8;              // rows per wave-wide 1 KB copy
  static constexpr int COPIES = BN / ROWS;           // copies per operand per tile
  static constexpr int STAGE = BN * D;               // bytes per operand

  __device__ static void issue(const AttnParams& p, int h, const TileInfo& ti, int8_t* stage, float* lks,
                               float* lvs, int wave, int lane) {
    const int64_t rs = int64_t(p.H) * D;
    const int8_t* gk = static_cast<const int8_t*>(p.cK) + int64_t(h) * D;
    const int8_t* gv = static_cast<const int8_t*>(p.cV) + int64_t(h) * D;
    for (int i = wave; i < COPIES; i += NW) {
      const int r0 = i * ROWS;
      const int r = r0 + lane / CH8;
      const int64_t base = int64_t(ti.start) * rs;
      const uint32_t off = uint32_t(int64_t(min(r, ti.cnt - 1)) * rs + 16 * (lane % CH8));
      copy_lds<16>(gk + base, off, stage + r0 * D);
      copy_lds<16>(gv + base, off, stage + STAGE + r0 * D);
    }
    if (wave < 2) {
      const float* sp = (wave == 0 ? p.cKs : p.cVs) + int64_t(ti.start) * p.H + h;
      copy_lds<4>(sp, uint32_t(min(lane, ti.cnt - 1) * p.H * 4), wave == 0 ? lks : lvs);
    }
  }

  // Called by the same wave after s_waitcnt vmcnt(0).
  __device__ static void widen(const int8_t* stage, uint16_t* lk, uint16_t* lv, int wave, int lane) {
    for (int i = wave; i < COPIES; i += NW) {
      const int r = i * ROWS + lane / CH8;
      const int c16 = lane % CH8;
#pragma unroll
      for (int op = 0; op < 2; ++op) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(stage + op * STAGE + i * ROWS * D + 16 * lane);
        uint16_t* dst = op ? lv : lk;
        *reinterpret_cast<u32x4*>(dst + r * D + 8 * swz<D>(r, 2 * c16)) =
            u32x4{code2_to_bf16x2<FMT>(q.x, 0), code2_to_bf16x2<FMT>(q.x, 2), code2_to_bf16x2<FMT>(q.y, 0),
                  code2_to_bf16x2<FMT>(q.y, 2)};
        *reinterpret_cast<u32x4*>(dst + r * D + 8 * swz<D>(r, 2 * c16 + 1)) =
            u32x4{code2_to_bf16x2<FMT>(q.z, 0), code2_to_bf16x2<FMT>(q.z, 2), code2_to_bf16x2<FMT>(q.w, 0),
                  code2_to_bf16x2<FMT>(q.w, 2)};
      }
    }
  }
};

// Order of the key tiles of a launch whose cached context is one run of rows (every
// cache without a shot sink): the (at most two) partial tiles -- the last tile of the
// run and of the own chunk -- come first, so that the long stretch of full tiles after
// them carries no masking code; then the full cache tiles, then the full own-chunk
// tiles.  Softmax attention does not depend on the order of its keys.
struct TileOrder1 {
  int n1, n2, np1, np2, ncache, nq, r0;
  __device__ explicit TileOrder1(const AttnParams& p)
      : ncache(p.nrun ? p.run_rows[0] : 0), nq(p.nq), r0(p.nrun ? p.run_row0[0] : 0) {
    n1 = (ncache + BN - 1) / BN;
    n2 = (nq + BN - 1) / BN;
    np1 = (ncache % BN) != 0;
    np2 = (nq % BN) != 0;
  }
  __device__ int npart() const { return np1 + np2; }
  __device__ int full1_end() const { return np1 + np2 + n1 - np1; }   // end of the full cache tiles
  __device__ int total() const { return n1 + n2; }
  __device__ TileInfo at(int j) const {
    TileInfo t;
    if (j < np1 + np2) {
      if (j == 0 && np1) {
        t.seg = 0;
        t.start = r0 + (n1 - 1) * BN;
        t.cnt = ncache - (n1 - 1) * BN;
      } else {
        t.seg = 1;
        t.start = (n2 - 1) * BN;
        t.cnt = nq - t.start;
      }
    } else if (j < full1_end()) {
      t.seg = 0;
      t.start = r0 + (j - np1 - np2) * BN;
      t.cnt = BN;
    } else {
      t.seg = 1;
      t.start = (j - full1_end()) * BN;
      t.cnt = BN;
    }
    return t;
  }
};

// General order of the key tiles (a shot sink can split the cached context).  The keys
// are the cached runs (up to kMaxRuns runs of rows of the slot array) and the own chunk; each is tiled on its own, so only the last tile of
// each may be partial.  The partial tiles come first, so that the long stretch of full
// tiles after them carries no masking code; then the full cache tiles run by run, then
// the full own-chunk tiles.  Softmax attention does not depend on the order of its keys.
// (All loops are unrolled over the run count so the tables stay in scalar registers.)
struct TileOrderN {
  int r0[kMaxRuns], rn[kMaxRuns], fc[kMaxRuns];   // first row, rows, full tiles per run
  int nq, np, nfc, pmask;   // own rows, partial tiles, full cache tiles, runs with a partial tile
  __device__ explicit TileOrderN(const AttnParams& p) : nq(p.nq), np(0), nfc(0), pmask(0) {
#pragma unroll
    for (int k = 0; k < kMaxRuns; ++k) {
      r0[k] = k < p.nrun ? p.run_row0[k] : 0;
      rn[k] = k < p.nrun ? p.run_rows[k] : 0;
      fc[k] = rn[k] / BN;
      nfc += fc[k];
      if (rn[k] % BN) {
        pmask |= 1 << k;
        ++np;
      }
    }
    if (nq % BN) ++np;
  }
  __device__ int npart() const { return np; }
  __device__ int full1_end() const { return np + nfc; }   // end of the full cache tiles
  __device__ int total() const { return np + nfc + nq / BN; }
  __device__ TileInfo at(int j) const {
    TileInfo t;
    if (j < np) {   // the j-th partial tile: runs in order, then the own chunk
      t.seg = 1;
      t.start = nq / BN * BN;
      t.cnt = nq % BN;
      int seen = 0;
#pragma unroll
      for (int k = 0; k < kMaxRuns; ++k)
        if ((pmask >> k) & 1) {
          if (seen == j) {
            t.seg = 0;
            t.start = r0[k] + fc[k] * BN;
            t.cnt = rn[k] - fc[k] * BN;
          }
          ++seen;
        }
    } else if (j < np + nfc) {
      const int jj = j - np;
      t.seg = 0;
      t.start = 0;
      t.cnt = BN;
      int base = 0;
#pragma unroll
      for (int k = 0; k < kMaxRuns; ++k) {
        if (jj >= base && jj < base + fc[k]) t.start = r0[k] + (jj - base) * BN;
        base += fc[k];
      }
    } else {
      t.seg = 1;
      t.start = (j - np - nfc) * BN;
      t.cnt = BN;
    }
    return t;
  }
};

template <int D, int NQB, int NW, bool KV8>
struct Attn {
  using G = Geo<D, NW>;
  bf16x8 qf[NQB][D / 16];
  f32x16 O[NQB][D / 32];
  float m[NQB], l[NQB];
  int g, r32, s16, h16;
  int kofs;        // K read: element offset of (row r32, chunk g), swizzled
  int vlo, vhi;    // V transpose reads: offsets of the lane's rows kA and kA + 8 (u = 0, e = 0)
  float c;

  // With the row swizzle c -> c ^ f(row), chunk 2 s + g of row r sits at 8 ((2 s) ^
  // (g ^ f(r))): the K read of step s is kofs ^ (16 s), and the V read of column block
  // e is vlo ^ (32 e).  Row blocks (32 b, Ku) and the buffer are immediate offsets.
  __device__ __forceinline__ void init_offsets(int lane) {
    g = lane >> 5;
    r32 = lane & 31;
    s16 = lane & 15;
    h16 = (lane >> 4) & 1;
    kofs = swz_row_base<D>(r32, g);
    const int kl = 4 * g + (s16 >> 2);
    const int cl = 2 * h16 + ((s16 & 3) >> 1);
    const int dhalf = 4 * (s16 & 1);
    vlo = swz_row_base<D>(kl, cl) + dhalf;
    vhi = swz_row_base<D>(kl + 8, cl) + dhalf;
  }

  // S^T = K Q^T for the 64 keys of a tile (two 32-key blocks).  MASK: keys >= cnt get
  // -inf; SCALED (int8 tile, when `scaled`): the per-key K scale multiplies its column.
  template <bool MASK, bool SCALED>
  __device__ __forceinline__ void scores(const uint16_t* lk, const float* lks, int cnt, bool scaled,
                                         f32x16 (&S)[NQB][2]) const {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) S[qb][0] = S[qb][1] = f32x16{};
    // Scaled (int8 / fp8) tiles: K fragments read two steps ahead of the MFMAs that use
    // them.  (Measured: that pays on the scaled tiles; on bf16 tiles the compiler's own
    // one-step order is faster.)
    constexpr int kLook = (SCALED && !MASK) ? 2 : 1;
    bf16x8 kf[kLook + 1][2];
    auto kread = [&](int s, bf16x8 (&f)[2]) __attribute__((always_inline)) {
      const int ko = kofs ^ (16 * s);
      f[0] = as_bf16x8(*reinterpret_cast<const u32x4*>(lk + ko));
      f[1] = as_bf16x8(*reinterpret_cast<const u32x4*>(lk + 32 * D + ko));
    };
    if constexpr (kLook > 1) {
#pragma unroll
      for (int s = 0; s < kLook; ++s) kread(s, kf[s]);
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if constexpr (kLook == 1) kread(s, kf[s & 1]);
      else if (s + kLook < D / 16) kread(s + kLook, kf[(s + kLook) % (kLook + 1)]);
      const bf16x8 (&f)[2] = kf[kLook == 1 ? (s & 1) : s % (kLook + 1)];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        S[qb][0] = mfma32(f[0], qf[qb][s], S[qb][0]);
        S[qb][1] = mfma32(f[1], qf[qb][s], S[qb][1]);
      }
    }
    if (SCALED && scaled) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 kscv = *reinterpret_cast<const f32x4*>(lks + 32 * b + 8 * i + 4 * g);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[qb][b][4 * i + jj] *= kscv[jj];
        }
    }
    if (MASK) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (32 * b + 8 * i + 4 * g + jj >= cnt) {
#pragma unroll
              for (int qb = 0; qb < NQB; ++qb) S[qb][b][4 * i + jj] = -__builtin_inff();
            }
    }
  }

  // Online softmax of one tile (base 2, lazy rescale) -> bf16 probabilities in the
  // B-operand layout of the P*V product.  SCALED: the per-key V scale multiplies P.
  template <bool SCALED>
  __device__ __forceinline__ void softmax(f32x16 (&S)[NQB][2], const float* lvs, bool scaled,
                                          bf16x8 (&P)[NQB][4]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = S[qb][0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[qb][b][v]);
      {  // lanes l and l ^ 32 hold the two halves of a query's keys: exchange in registers
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
      }
      if (__builtin_amdgcn_ballot_w64(mx > m[qb] + kLazyThreshold)) {
        const float mnew = fmaxf(m[qb], mx);
        const float alpha = fast_exp2(m[qb] - mnew);
        m[qb] = mnew;
        l[qb] *= alpha;
#pragma unroll
        for (int e = 0; e < D / 32; ++e) O[qb][e] *= alpha;
      }
      const float mq = m[qb];
      float rsum = 0.0f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          S[qb][b][v] = fast_exp2(__builtin_fmaf(S[qb][b][v], c, -mq));
          if (SCALED && scaled) rsum += S[qb][b][v];
        }
      if (SCALED && scaled) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 vscv = *reinterpret_cast<const f32x4*>(lvs + 32 * b + 8 * i + 4 * g);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[qb][b][4 * i + jj] *= vscv[jj];
          }
      }
      // Unscaled tiles: the row sum is taken over the bf16 probabilities that P*V uses
      // (two per dot2), so the normalised weights sum to one exactly as applied.
      // Scaled tiles sum the fp32 probabilities before the V scale (above).
      const bool sum_packed = !(SCALED && scaled);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = u >> 1, v0 = 8 * (u & 1);
        u32x4 w;
        w.x = pack_bf16x2(S[qb][b][v0 + 0], S[qb][b][v0 + 1]);
        w.y = pack_bf16x2(S[qb][b][v0 + 2], S[qb][b][v0 + 3]);
        w.z = pack_bf16x2(S[qb][b][v0 + 4], S[qb][b][v0 + 5]);
        w.w = pack_bf16x2(S[qb][b][v0 + 6], S[qb][b][v0 + 7]);
        P[qb][u] = as_bf16x8(w);
        if (sum_packed) {
          rsum = dot2_ones(w.x, rsum);
          rsum = dot2_ones(w.y, rsum);
          rsum = dot2_ones(w.z, rsum);
          rsum = dot2_ones(w.w, rsum);
        }
      }
      l[qb] += rsum;
    }
  }

  // V^T operand of column block e, step u.  B slot t of step u holds key 32 (u>>1) +
  // 16 (u&1) + 8 (t>>2) + 4 g + (t&3).  The transpose read gives lane s16 of a 16-lane
  // group element (s16 & 3) of the rows addressed by lanes (s16 >> 2) + 4 k, k = 0..3:
  // lane s16 therefore addresses key row kA + (s16 >> 2), columns d0 + 4 (s16 & 3) .. + 3
  // (the row swizzle depends on row & 15 only, so row blocks are immediate offsets).
  __device__ __forceinline__ bf16x8 v_operand(const uint16_t* lv, int e, int u) const {
    const int ku = (32 * (u >> 1) + 16 * (u & 1)) * D;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lv + ku + (vlo ^ (32 * e))));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lv + ku + (vhi ^ (32 * e))));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // O^T += V^T P^T over the 64 keys of a tile.  Key-step-major: the first MFMAs need
  // only the first 8 probabilities, so they can start while later exps are computed.
  // ORDERED: the V^T fragments of key step u + 1 are read before the MFMAs of step u
  // are issued, an order pinned through the scheduler with sched_group_barrier (left
  // to itself it reads each fragment just before its MFMA and waits for it there).
  // Used on the bf16 tiles; on the scaled tiles the extra live fragments cost more.
  template <bool ORDERED>
  __device__ __forceinline__ void pv(const uint16_t* lv, const bf16x8 (&P)[NQB][4]) {
    if constexpr (ORDERED) {
      bf16x8 vf[2][D / 32];
#pragma unroll
      for (int e = 0; e < D / 32; ++e) vf[0][e] = v_operand(lv, e, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u + 1 < 4) {
#pragma unroll
          for (int e = 0; e < D / 32; ++e) vf[(u + 1) & 1][e] = v_operand(lv, e, u + 1);
        }
#pragma unroll
        for (int e = 0; e < D / 32; ++e)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) O[qb][e] = mfma32(vf[u & 1][e], P[qb][u], O[qb][e]);
      }
      // groups in issue order (0x100 = LDS reads, 0x008 = MFMAs): reads of steps 0 and
      // 1, MFMAs of step 0, reads of step 2, MFMAs of step 1, reads of step 3, MFMAs of
      // steps 2 and 3
      __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NQB * D / 32, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NQB * D / 32, 0);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < D / 32; ++e) {
          const bf16x8 vf = v_operand(lv, e, u);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) O[qb][e] = mfma32(vf, P[qb][u], O[qb][e]);
        }
    }
  }

  // Probabilities of a full unscaled tile against running max mq, packed to bf16 in
  // the P*V operand layout; returns the lane's sum of the packed values (the weights
  // P*V applies).
  __device__ __forceinline__ float exp_pack(const f32x16 (&S)[2], float mq, bf16x8 (&P)[4]) const {
    float part[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = u >> 1, v0 = 8 * (u & 1);
      float e[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) e[t] = fast_exp2(__builtin_fmaf(S[b][v0 + t], c, -mq));
      u32x4 w;
      w.x = pack_bf16x2(e[0], e[1]);
      w.y = pack_bf16x2(e[2], e[3]);
      w.z = pack_bf16x2(e[4], e[5]);
      w.w = pack_bf16x2(e[6], e[7]);
      P[u] = as_bf16x8(w);
      part[u] = dot2_ones(w.w, dot2_ones(w.z, dot2_ones(w.y, dot2_ones(w.x, 0.0f))));
    }
    return (part[0] + part[1]) + (part[2] + part[3]);
  }

  // Full unscaled tile with the probabilities first taken against the running max as it
  // stands.  They are non-negative, so all of a lane's probabilities are at most 2^8
  // exactly when its tile sum is; then the tile needs no new max (the same bound the
  // lazy rescale keeps).  Otherwise (a score more than 8 above the running max, or the
  // first tile of a walk, where the max is -inf) the scores are recomputed from the K
  // tile, still in LDS, the running max is raised to the tile's max and O and l are
  // rescaled before the probabilities are taken again.  The common case skips the
  // per-tile max and its exchange between the two lanes of a query.  (Scaled int8 /
  // fp8 tiles keep softmax(): there the extra scale work ate the gain.)
  __device__ __forceinline__ void tile_spec(const uint16_t* lk, const uint16_t* lv) {
    constexpr float kBound = float(1 << int(kLazyThreshold));
    f32x16 S[NQB][2];
    bf16x8 P[NQB][4];
    scores<false, false>(lk, nullptr, BN, false, S);
    float rsum[NQB];
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      rsum[qb] = exp_pack(S[qb], m[qb], P[qb]);
      over |= !(rsum[qb] <= kBound);
    }
    if (__builtin_amdgcn_ballot_w64(over)) {
      // an offset the compiler cannot see through: the K fragments are read again here
      // instead of being held in registers across the exponentials for this rare case
      int z = 0;
      asm volatile("" : "+s"(z));
      scores<false, false>(lk + z, nullptr, BN, false, S);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float mx = S[qb][0][0];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[qb][b][v]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        const float mnew = fmaxf(m[qb], fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c);
        const float alpha = fast_exp2(m[qb] - mnew);
        m[qb] = mnew;
        l[qb] *= alpha;
#pragma unroll
        for (int e = 0; e < D / 32; ++e) O[qb][e] *= alpha;
        rsum[qb] = exp_pack(S[qb], mnew, P[qb]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) l[qb] += rsum[qb];
    pv<true>(lv, P);
  }

  // One whole tile from LDS: scores, softmax, P*V.
  template <bool MASK, bool SCALED>
  __device__ __forceinline__ void tile(const uint16_t* lk, const uint16_t* lv, const float* lks, const float* lvs,
                                       int cnt, bool scaled = SCALED) {
    if constexpr (kSpecSoftmax && !MASK && !SCALED) {
      tile_spec(lk, lv);
    } else {
      f32x16 S[NQB][2];
      bf16x8 P[NQB][4];
      scores<MASK, SCALED>(lk, lks, cnt, scaled, S);
      softmax<SCALED>(S, lvs, scaled, P);
      pv<false>(lv, P);
    }
  }

  // Normalise and store O (lane: query r32, d = 32 e + 8 i + 4 g + [0, 4)).
  __device__ __forceinline__ void store(uint16_t* out, int q0, int nq, int64_t rs, int h) const {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float lt = l[qb] + __shfl_xor(l[qb], 32);
      const float inv = 1.0f / lt;
      const int row = q0 + 32 * qb + r32;
      if (row < nq) {
        uint16_t* dst = out + int64_t(row) * rs + int64_t(h) * D;
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

  // Un-normalised O, reference max m and row sum l of this wave's rows, fp32, into a
  // partial-result slot: O at [row][D], then m[rows], then l[rows] (row = the row
  // within the block).  Device-coherent stores (they bypass the non-coherent caches),
  // so another workgroup's device-coherent loads see them without a cache flush.
  __device__ __forceinline__ void store_partial(float* slot, int rows, int wave) const {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int row = wave * 32 * NQB + 32 * qb + r32;
      const float lt = l[qb] + __shfl_xor(l[qb], 32);
      const __amdgpu_buffer_rsrc_t rsrc = coherent_rsrc(slot);
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          coherent_store4(rsrc, 4u * uint32_t(row * D + 32 * e + 8 * i + 4 * g),
                          f32x4{O[qb][e][4 * i], O[qb][e][4 * i + 1], O[qb][e][4 * i + 2], O[qb][e][4 * i + 3]});
      if (g == 0) {
        coherent_store(slot + rows * D + row, m[qb]);
        coherent_store(slot + rows * D + rows + row, lt);
      }
    }
  }

  // Combine this wave's own piece (registers) with the partial results of the other
  // pieces of the block over disjoint key sets:
  //   M = max_i m_i,  O = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i,
  // then store.  The same identity as the running rescale inside one piece.  The sums
  // run over the pieces in block order (head piece, then the tail pieces) whichever
  // piece does the merge, so the result does not depend on which one arrived last.
  //   slot_k: partial of piece k (unused for k == own); n: pieces (2 or 3)
  __device__ __forceinline__ void merge_store(const float* s0, const float* s1, const float* s2, int own, int n,
                                              int rows, int wave, uint16_t* out, int q0, int nq, int64_t rs,
                                              int h) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int row = wave * 32 * NQB + 32 * qb + r32;
      const float lown = l[qb] + __shfl_xor(l[qb], 32);
      float mk[3], lk[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float* sl = k == 0 ? s0 : k == 1 ? s1 : s2;
        const bool mem = k < n && k != own;
        mk[k] = k == own ? m[qb] : (mem ? coherent_load(sl + rows * D + row) : -__builtin_inff());
        lk[k] = k == own ? lown : (mem ? coherent_load(sl + rows * D + rows + row) : 0.0f);
      }
      const float M = fmaxf(fmaxf(mk[0], mk[1]), mk[2]);
      float f[3];
      float L = 0.0f;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        f[k] = k < n ? fast_exp2(mk[k] - M) : 0.0f;
        if (k < n) L += f[k] * lk[k];
      }
      const __amdgpu_buffer_rsrc_t r0 = coherent_rsrc(s0), r1 = coherent_rsrc(s1), r2 = coherent_rsrc(s2);
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t off = 4u * uint32_t(row * D + 32 * e + 8 * i + 4 * g);
          const f32x4 mine = f32x4{O[qb][e][4 * i], O[qb][e][4 * i + 1], O[qb][e][4 * i + 2], O[qb][e][4 * i + 3]};
          const f32x4 x0 = own == 0 ? mine : coherent_load4(r0, off);
          const f32x4 x1 = own == 1 ? mine : coherent_load4(r1, off);
          f32x4 acc = x0 * f[0] + x1 * f[1];
          if (n > 2) acc = acc + (own == 2 ? mine : coherent_load4(r2, off)) * f[2];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) O[qb][e][4 * i + jj] = acc[jj];
        }
      // store() halves the row sum across the lane pair: hand it half of L per lane
      l[qb] = 0.5f * L;
    }
    store(out, q0, nq, rs, h);
  }

  // Q^T fragments (MFMA B operand): lane holds query r32, d = 16 s + 8 g + [0, 8).
  __device__ __forceinline__ void load_q(const uint16_t* Q, int q0, int nq, int64_t rs, int h, float c_) {
    c = c_;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int row = q0 + 32 * qb + r32;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        u32x4 w = {0, 0, 0, 0};
        if (row < nq) w = *reinterpret_cast<const u32x4*>(Q + int64_t(row) * rs + int64_t(h) * D + 16 * s + 8 * g);
        qf[qb][s] = as_bf16x8(w);
      }
      m[qb] = -__builtin_inff();
      l[qb] = 0.0f;
#pragma unroll
      for (int e = 0; e < D / 32; ++e) O[qb][e] = f32x16{};
    }
    // Wait for the Q fragments here, with a wait the compiler sees: their first use is
    // inside the key walk, where it would otherwise place a memory-counter wait at the
    // first MFMAs of every tile -- which also waits for the next tile's copies.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  }
};

// Per-XCD work plan of a split launch: blocks [b0, b0 + nb) run on this XCD, one
// workgroup each for their first J - t tiles; ns spare workgroups take the tails, spare
// s the tail units [s L, (s + 1) L) of the XCD (unit = one tile of one block's tail,
// block-major).  L >= t, so a tail meets at most two spares and a block has at most
// three pieces.
struct XcdPlan {
  int b0 = 0, nb = 0, ns = 0, t = 0, L = 0;
  XcdPlan() = default;
  __host__ __device__ XcdPlan(const Split& sp, int x) {
    b0 = x * sp.B / NXCD;
    nb = (x + 1) * sp.B / NXCD - b0;
    ns = sp.per_xcd - nb;
    // heads walk J - t tiles; a spare walks about nb t / ns tiles over about nb / ns + 1
    // pieces, each costing ~kPieceTiles tiles of set-up and hand-over: equal times at
    // t = J ns / (nb + ns) - kPieceTiles.
    t = ns > 0 ? max(0, sp.J * ns / (nb + ns) - kPieceTiles) : 0;
    L = t ? (nb * t + ns - 1) / ns : 0;
  }
  __host__ __device__ int first_spare(int b) const { return b * t / L; }
  __host__ __device__ int n_tail(int b) const { return ((b + 1) * t - 1) / L - b * t / L + 1; }
};

template <int D, int NQB, int NW, int MINB, int KVQ, bool RUNS>
__global__ __launch_bounds__(64 * NW, MINB) void attn_kernel(const AttnParams p, const Split sp) {
  using G = Geo<D, NW>;
  // Two buffers per operand as separate LDS objects: the buffer parity is a compile-time
  // constant at every access, which lets the compiler see that the copy into the next
  // buffer does not alias the reads of the current one (no wait before the reads).
  __shared__ __attribute__((aligned(1024))) uint16_t sm_k0[G::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sm_k1[G::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sm_v0[G::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sm_v1[G::TILE];
  constexpr bool KV8 = KVQ != kKvBf16;   // quantised cache (int8 or fp8 codes)
  __shared__ __attribute__((aligned(16))) float sm_ks0[KV8 ? BN : 1];
  __shared__ __attribute__((aligned(16))) float sm_ks1[KV8 ? BN : 1];
  __shared__ __attribute__((aligned(16))) float sm_vs0[KV8 ? BN : 1];
  __shared__ __attribute__((aligned(16))) float sm_vs1[KV8 ? BN : 1];
  __shared__ __attribute__((aligned(1024))) int8_t sm_stage[KV8 ? 2 * QTile<D, NW, KVQ>::STAGE : 16];
  __shared__ int sm_last;
  constexpr int ROWS = NW * 32 * NQB;   // query rows per block

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t rs = int64_t(p.H) * D;

  Attn<D, NQB, NW, KV8> A;
  A.init_offsets(lane);

  // RUNS: the cached context may be several runs of slots (shot sink)
  const std::conditional_t<RUNS, TileOrderN, TileOrder1> order(p);
  const int ntiles = order.total();
  uint32_t loff[Geo<D, NW>::DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < Geo<D, NW>::DMA_PER_WAVE; ++i) loff[i] = dma_lane_offset<D, NW>(rs, wave, lane, i);

  // One piece: block blk (head, query tile) over key tiles [ja, jb) of the tile order,
  // one of the block's npc pieces.  A whole block stores its output; otherwise the piece
  // leaves a partial result in its slot and the last piece of the block to arrive
  // merges them all.
  auto piece = [&](int blk, int ja, int jb, int npc, int slot) __attribute__((always_inline)) {
    const int h = blk / sp.n_qtiles;
    const int q0 = (blk % sp.n_qtiles) * ROWS + wave * (32 * NQB);
    const int jend = jb;
    const uint16_t* ck = KV8 ? nullptr : static_cast<const uint16_t*>(p.cK) + int64_t(h) * D;
    const uint16_t* cv = KV8 ? nullptr : static_cast<const uint16_t*>(p.cV) + int64_t(h) * D;
    const uint16_t* kc = p.Kc + int64_t(h) * D;
    const uint16_t* vc = p.Vc + int64_t(h) * D;
    A.load_q(p.Q, q0, p.nq, rs, h, p.c);

    // Loads of tile j into buffer PB.  int8 tiles go to the staging area first and are
    // widened by finish().  Returns true when a widening is pending.
    auto issue = [&](auto pb, int j) __attribute__((always_inline)) -> bool {
      constexpr int PB = decltype(pb)::value;
      const TileInfo t = order.at(j);
      if (KV8 && t.seg == 0) {
        QTile<D, NW, KVQ>::issue(p, h, t, sm_stage, PB ? sm_ks1 : sm_ks0, PB ? sm_vs1 : sm_vs0, wave, lane);
        return true;
      }
      dma_tile<D, NW>(t.seg == 0 ? ck : kc, t.seg == 0 ? cv : vc, rs, t, PB ? sm_k1 : sm_k0, PB ? sm_v1 : sm_v0,
                      wave, lane);
      return false;
    };
    // A full bf16 tile (every tile after the partial ones, except int8 cache tiles).
    auto issue_full = [&](auto pb, int j) __attribute__((always_inline)) {
      constexpr int PB = decltype(pb)::value;
      const TileInfo t = order.at(j);
      const int64_t base = int64_t(t.start) * rs;
      dma_full<D, NW>((t.seg == 0 ? ck : kc) + base, (t.seg == 0 ? cv : vc) + base, loff, PB ? sm_k1 : sm_k0,
                      PB ? sm_v1 : sm_v0, wave);
    };
    auto finish = [&](auto pb, bool pending) __attribute__((always_inline)) {
      constexpr int PB = decltype(pb)::value;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (KV8 && pending) QTile<D, NW, KVQ>::widen(sm_stage, PB ? sm_k1 : sm_k0, PB ? sm_v1 : sm_v0, wave, lane);
      __syncthreads();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // Full tiles: prefetch the next tile into the other buffer, compute this one.  The
    // buffer parity is a template argument so LDS accesses name a fixed buffer.
    // KIND 1: int8 cache tiles (scaled), 2: bf16 tiles (cache or own chunk).
    auto step = [&](auto pb, auto kind, int j) __attribute__((always_inline)) {
      constexpr int PB = decltype(pb)::value;
      constexpr int KIND = decltype(kind)::value;
      bool pend = false;
      if (j + 1 < jend) {
        if (KIND == 2 || !KV8) {
          issue_full(std::integral_constant<int, PB ^ 1>{}, j + 1);
        } else {
          pend = issue(std::integral_constant<int, PB ^ 1>{}, j + 1);
        }
      }
      A.template tile<false, KIND == 1>(PB ? sm_k1 : sm_k0, PB ? sm_v1 : sm_v0, PB ? sm_ks1 : sm_ks0,
                                        PB ? sm_vs1 : sm_vs0, BN);
      finish(std::integral_constant<int, PB ^ 1>{}, pend);
    };
    auto run = [&](auto kind, int j, int end) __attribute__((always_inline)) -> int {
      if (j < end && (j & 1)) step(I1{}, kind, j++);
      for (; j + 1 < end; j += 2) {
        step(I0{}, kind, j);
        step(I1{}, kind, j + 1);
      }
      if (j < end) step(I0{}, kind, j++);
      return j;
    };

    if (ja & 1) finish(I1{}, issue(I1{}, ja));
    else finish(I0{}, issue(I0{}, ja));
    int j = ja;
    // Partial tiles (at most two): one generic masked path with run-time buffer choice.
    for (; j < min(jb, order.npart()); ++j) {
      bool pend = false;
      if (j + 1 < jb) pend = (j & 1) ? issue(I0{}, j + 1) : issue(I1{}, j + 1);
      const TileInfo t = order.at(j);
      const bool odd = j & 1;
      A.template tile<true, KV8>(odd ? sm_k1 : sm_k0, odd ? sm_v1 : sm_v0, odd ? sm_ks1 : sm_ks0,
                                 odd ? sm_vs1 : sm_vs0, t.cnt, KV8 && t.seg == 0);
      if (j & 1) finish(I0{}, pend);
      else finish(I1{}, pend);
    }
    if (KV8) j = run(std::integral_constant<int, 1>{}, j, min(jb, order.full1_end()));
    run(std::integral_constant<int, 2>{}, j, jb);

    if (npc == 1) {
      A.store(p.out, q0, p.nq, rs, h);
      return;
    }
    // The partials go out with device-coherent stores; waiting for them to complete
    // before the arrival count orders them before it for every observer.  The last
    // piece reads the others with device-coherent loads after seeing the count.  No
    // cache is flushed or invalidated (that would evict the key/value tiles the other
    // workgroups of the XCD are streaming).
    // A piece that finds every other piece already counted is the last one: it merges
    // from its registers without leaving a partial (the common case for the head piece,
    // which has the longest walk).
    const int64_t slot_floats = split_slot_floats(D, ROWS);
    if (tid == 0) sm_last = coherent_load(sp.cnt + blk) == npc - 1;
    __syncthreads();
    if (!sm_last) {
      A.store_partial(sp.ws + slot * slot_floats, ROWS, wave);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) sm_last = atomicAdd(sp.cnt + blk, 1) == npc - 1;
      __syncthreads();
    }
    if (sm_last) {
      // the block's pieces in order: blk (head piece), B + 2 blk + k (tail pieces)
      const int own = slot == blk ? 0 : slot - (sp.B + 2 * blk) + 1;
      A.merge_store(sp.ws + int64_t(blk) * slot_floats, sp.ws + int64_t(sp.B + 2 * blk) * slot_floats,
                    sp.ws + int64_t(sp.B + 2 * blk + 1) * slot_floats, own, npc, ROWS, wave, p.out, q0, p.nq, rs,
                    h);
      if (tid == 0) coherent_store(sp.cnt + blk, 0);   // ready for the next call on the stream
    }
    __syncthreads();
  };

  // The pieces of this workgroup.  Plain launch: one workgroup per block (XCD-aware
  // numbering: hardware deals block ids round-robin over the XCDs; each XCD gets a
  // contiguous range of blocks, so query tiles of one head share its L2 while they
  // stream the same keys).  Split launch: one workgroup per CU; on each XCD workgroup
  // i < nb walks the first J - t tiles of its block (in step with the others, as
  // above) and the ns = per_xcd - nb spare workgroups share the blocks' last t tiles
  // ("tails"), so every CU gets about the same number of tiles.
  const int J = ntiles;
  if (!sp.on || int(blockIdx.x) / NXCD < XcdPlan(sp, blockIdx.x % NXCD).nb) {
    int blk, jb = J, npc = 1;
    if (!sp.on) {
      const int per_xcd = (sp.B + NXCD - 1) / NXCD;
      blk = (blockIdx.x % NXCD) * per_xcd + blockIdx.x / NXCD;
      if (blk >= sp.B) return;
    } else {
      const XcdPlan xp(sp, blockIdx.x % NXCD);
      const int i = blockIdx.x / NXCD;
      blk = xp.b0 + i;
      jb = J - xp.t;
      npc = xp.t ? 1 + xp.n_tail(i) : 1;
    }
    piece(blk, 0, jb, npc, blk);
    return;
  }
  const XcdPlan xp(sp, blockIdx.x % NXCD);
  const int sidx = int(blockIdx.x) / NXCD - xp.nb;
  if (sidx >= xp.ns || xp.t == 0) return;
  const int u1 = min((sidx + 1) * xp.L, xp.nb * xp.t);
  for (int u = sidx * xp.L; u < u1;) {
    const int bl = u / xp.t;
    const int e = min(u1, (bl + 1) * xp.t);
    const int blk = xp.b0 + bl;
    const int ja = J - xp.t + (u - bl * xp.t);
    piece(blk, ja, ja + (e - u), 1 + xp.n_tail(bl), sp.B + 2 * blk + (xp.first_spare(bl) == sidx ? 0 : 1));
    u = e;
  }
}


template <int D, int NQB, int NW, int KVQ, int MINB = 1>
hipError_t launch_t(const AttnParams& p, hipStream_t s) {
  const int rows = NW * 32 * NQB;
  Split sp{};
  sp.n_qtiles = (p.nq + rows - 1) / rows;
  sp.B = sp.n_qtiles * p.H;
  sp.J = (p.nq + BN - 1) / BN;
  for (int k = 0; k < p.nrun; ++k) sp.J += (p.run_rows[k] + BN - 1) / BN;
  sp.ws = p.ws;
  sp.cnt = p.cnt;
  // Split when the blocks leave CUs idle, every XCD has at least as many blocks as spare
  // workgroups (so L >= t) and the walk is long enough to be worth a merge.
  bool on = p.ws && p.cnt && p.n_cu % NXCD == 0 && sp.B < p.n_cu && sp.J >= 32 &&
            split_slot_floats(D, rows) * 3 * int64_t(p.n_cu) <= p.ws_floats;
  if (on) {
    sp.per_xcd = p.n_cu / NXCD;
    for (int x = 0; x < NXCD && on; ++x) {
      const XcdPlan xp(sp, x);
      on = xp.nb >= 1 && xp.nb >= xp.ns && (xp.t == 0 || xp.L >= xp.t);
    }
  }
  sp.on = on;
  const int grid = on ? p.n_cu : (sp.B + NXCD - 1) / NXCD * NXCD;
  if (p.nrun > 1)
    hipLaunchKernelGGL((attn_kernel<D, NQB, NW, MINB, KVQ, true>), dim3(grid), dim3(64 * NW), 0, s, p, sp);
  else
    hipLaunchKernelGGL((attn_kernel<D, NQB, NW, MINB, KVQ, false>), dim3(grid), dim3(64 * NW), 0, s, p, sp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int D, int kv_fmt, hipStream_t s) {
// 8 waves of 32 query rows: two waves per SIMD, so one wave's softmax overlaps the
// other's MFMAs and every accumulator fits the 256 architected VGPRs.
  const bool big = p.nq > 4 * 32;
  if (D == 128) {
    switch (kv_fmt) {
      case kKvBf16: return big ? launch_t<128, 1, 8, kKvBf16>(p, s) : launch_t<128, 1, 4, kKvBf16>(p, s);
      case kKvInt8: return big ? launch_t<128, 1, 8, kKvInt8>(p, s) : launch_t<128, 1, 4, kKvInt8>(p, s);
      case kKvFp8: return big ? launch_t<128, 1, 8, kKvFp8>(p, s) : launch_t<128, 1, 4, kKvFp8>(p, s);
    }
  } else if (D == 64) {
    switch (kv_fmt) {
      case kKvBf16: return big ? launch_t<64, 2, 4, kKvBf16>(p, s) : launch_t<64, 1, 4, kKvBf16>(p, s);
      case kKvInt8: return big ? launch_t<64, 2, 4, kKvInt8>(p, s) : launch_t<64, 1, 4, kKvInt8>(p, s);
      case kKvFp8: return big ? launch_t<64, 2, 4, kKvFp8>(p, s) : launch_t<64, 1, 4, kKvFp8>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ll
