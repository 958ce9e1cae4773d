// split_plan.h -- work plan of a split attention launch (host and device code).
//
// When an attention launch has fewer blocks (head x query tile) than compute units,
// it runs one workgroup per CU and shares the key walk: on each XCD (workgroup id
// mod 8, how the hardware deals workgroups), the nb blocks of that XCD each walk
// their first J - t key tiles with one workgroup ("head pieces"), and the ns spare
// workgroups of the XCD walk the blocks' last t tiles ("tails"), spare s taking the
// tail units [s L, (s + 1) L) (unit = one tile of one block's tail, block-major).
// Each piece of a block that is not the whole block leaves a partial result (O, m, l)
// in a slot of the work area; the last piece to arrive merges them.
//
// Slots: head piece of block b -> slot b; tail pieces of XCD x -> slots
// B + x (per_xcd - 1) + (tail pieces of the XCD's earlier blocks) + k, k = 0, 1.
// An XCD has at most nb + ns - 1 = per_xcd - 1 tail pieces (each spare boundary
// inside a block's tail adds one piece to the nb blocks' first ones), so a launch
// uses fewer than B + CUs <= 2 CUs slots.
//
// Builds with plain g++ (no HIP) so that the plan can be checked on the host.
#pragma once

#include <cstdint>

#ifdef __HIPCC__
// always inlined: in the attention kernel the piece body is inlined into for_each_piece
#define LL_HD __host__ __device__ __attribute__((always_inline))
#else
#define LL_HD
#endif

namespace ll {

constexpr int kXcds = 8;
constexpr int kPieceTiles = 12;   // per-piece set-up and hand-over cost, in tiles

// Work description of one attention launch.
struct Split {
  int B;          // blocks = heads x query tiles
  int n_qtiles;
  int J;          // key tiles per block
  int on;         // 1: one workgroup per CU, tails of the key walk shared (per XCD)
  int per_xcd;    // workgroups per XCD when on
  float* ws;      // partial-result slots
  int* cnt;       // per-block arrival counters (zero between launches)
};

// Work-area slots a split launch may use, for a device with n_cu compute units.
inline LL_HD int64_t split_slots(int n_cu) { return 2 * int64_t(n_cu); }

// Per-XCD work plan: blocks [b0, b0 + nb) run on this XCD, one workgroup each for
// their first J - t tiles; ns spare workgroups take the tails.  L >= t, so a tail
// meets at most two spares and a block has at most three pieces.
struct XcdPlan {
  int x = 0, b0 = 0, nb = 0, ns = 0, t = 0, L = 0, per_xcd = 0, B = 0;
  XcdPlan() = default;
  LL_HD XcdPlan(const Split& sp, int xcd) {
    x = xcd;
    B = sp.B;
    per_xcd = sp.per_xcd;
    b0 = x * sp.B / kXcds;
    nb = (x + 1) * sp.B / kXcds - b0;
    ns = sp.per_xcd - nb;
    // heads walk J - t tiles; a spare walks about nb t / ns tiles over about nb / ns + 1
    // pieces, each costing ~kPieceTiles tiles of set-up and hand-over: equal times at
    // t = J ns / (nb + ns) - kPieceTiles.
    t = ns > 0 ? (sp.J * ns / (nb + ns) - kPieceTiles > 0 ? sp.J * ns / (nb + ns) - kPieceTiles : 0) : 0;
    L = t ? (nb * t + ns - 1) / ns : 0;
  }
  LL_HD int first_spare(int b) const { return b * t / L; }
  LL_HD int n_tail(int b) const { return ((b + 1) * t - 1) / L - b * t / L + 1; }
  // First slot of local block bl's tail pieces.
  LL_HD int tail_base(int bl) const {
    int s = B + x * (per_xcd - 1);
    for (int b = 0; b < bl; ++b) s += n_tail(b);
    return s;
  }
};

// One piece of work: block blk over key tiles [ja, jb) of the block's tile order,
// one of the block's npc pieces, leaving its partial (if any) in slot `slot`; the
// block's tail pieces use slots tail0 and tail0 + 1.
struct Piece {
  int blk, ja, jb, npc, slot, tail0;
};

// Call f(piece) for every piece workgroup `wg` of a launch runs, in order.  Without
// the split every block is one workgroup: hardware deals workgroup ids round-robin
// over the XCDs, so each XCD gets a contiguous range of blocks (query tiles of one
// head share its L2 while they stream the same keys).
template <class F>
LL_HD void for_each_piece(const Split& sp, int wg, F&& f) {
  const int J = sp.J;
  // one call site for the block-sized piece (no split, or a head piece), one for the
  // tails: the piece body is large and inlined at each
  Piece whole{-1, 0, J, 1, 0, 0};
  XcdPlan xp;
  int i = 0;
  if (!sp.on) {
    const int per_xcd = (sp.B + kXcds - 1) / kXcds;
    whole.blk = (wg % kXcds) * per_xcd + wg / kXcds;
    whole.slot = whole.blk;
    if (whole.blk >= sp.B) whole.blk = -1;
  } else {
    xp = XcdPlan(sp, wg % kXcds);
    i = wg / kXcds;
    if (i < xp.nb) {
      whole.blk = whole.slot = xp.b0 + i;
      whole.jb = J - xp.t;
      whole.npc = xp.t ? 1 + xp.n_tail(i) : 1;
      whole.tail0 = xp.t ? xp.tail_base(i) : 0;
    }
  }
  if (!sp.on || i < xp.nb) {
    if (whole.blk >= 0) f(whole);
    return;
  }
  const int sidx = i - xp.nb;
  if (sidx >= xp.ns || xp.t == 0) return;
  const int u1 = (sidx + 1) * xp.L < xp.nb * xp.t ? (sidx + 1) * xp.L : xp.nb * xp.t;
  for (int u = sidx * xp.L; u < u1;) {
    const int bl = u / xp.t;
    const int e = u1 < (bl + 1) * xp.t ? u1 : (bl + 1) * xp.t;
    const int ja = J - xp.t + (u - bl * xp.t);
    const int tb = xp.tail_base(bl);
    f(Piece{xp.b0 + bl, ja, ja + (e - u), 1 + xp.n_tail(bl), tb + (xp.first_spare(bl) == sidx ? 0 : 1), tb});
    u = e;
  }
}

// Decide whether a launch of B blocks with J key tiles per block splits its walk on a
// device with n_cu CUs, given ws_slots work-area slots: when the blocks leave CUs idle,
// every XCD has at least as many blocks as spare workgroups (so L >= t) and the walk is
// long enough to be worth a merge.
inline LL_HD bool plan_split(Split& sp, int n_cu, int64_t ws_slots) {
  bool on = sp.ws && sp.cnt && n_cu % kXcds == 0 && sp.B < n_cu && sp.J >= 32 && split_slots(n_cu) <= ws_slots;
  if (on) {
    sp.per_xcd = n_cu / kXcds;
    for (int x = 0; x < kXcds && on; ++x) {
      const XcdPlan xp(sp, x);
      on = xp.nb >= 1 && xp.nb >= xp.ns && (xp.t == 0 || xp.L >= xp.t);
    }
  }
  sp.on = on;
  return on;
}

}  // namespace ll
