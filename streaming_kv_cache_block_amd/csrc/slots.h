// slots.h -- host-side slot arithmetic of the sink + window KV cache (header-only, C++17).
//
// Policy ("LongLive: Real-time Interactive Long Video Generation" explainer, dpshk.com,
// §五 and §六; techwalker.com LONGLIVE article, §六): a layer keeps the first S frames
// permanently (sink) and the K/V of the most recent W frames (window); anything older
// is evicted.  Optional shot sink (LongLive-2.0 explainer, wmrh.cn, §16: a global sink
// for every shot plus a sink of the current shot): the first Ss frames of the shot that
// started at frame fs stay visible for the whole shot.  The library stores this in
// S + Ss + W fixed slots:
//
//   global sink  slot f                          for f < S
//   shot sink    slot S + (f - fs)               for f >= S, fs <= f < fs + Ss
//   window ring  slot S + Ss + (f - S) mod W     for f >= S, W > 0
//
// A shot-sink frame is stored in both its shot slot and its ring slot (one writer per
// slot).  The cached part of a chunk's context (sink, shot sink, window as a set) is
// then at most three runs of slots: [0, min(S, f0)), the shot frames that have left
// the window, and the occupied ring slots [S + Ss, S + Ss + min(W, f0 - S)), each
// scanned in physical order (softmax attention does not depend on key order).
// Without a shot sink the occupied slots are exactly the prefix [0, min(f0, S + W)).
//
// Builds with plain g++ (no HIP) for host-only tests.  With LL_DEBUG defined every
// slot index and plan entry is bounds-checked (abort with a message on failure).
#pragma once

#include <algorithm>
#include <cstdint>
#include <vector>

#ifdef LL_DEBUG
#include <cstdio>
#include <cstdlib>
#define LL_CHECK(cond)                                                                      \
  do {                                                                                      \
    if (!(cond)) {                                                                          \
      std::fprintf(stderr, "LL_DEBUG check failed: %s (%s:%d)\n", #cond, __FILE__, __LINE__); \
      std::abort();                                                                         \
    }                                                                                       \
  } while (0)
#else
#define LL_CHECK(cond) ((void)0)
#endif

namespace ll {

struct WriteEntry {
  int src;        // frame index within the caller's tensor
  int slot;       // destination slot
  int64_t frame;  // absolute frame id stored in the slot
};

struct Layout {
  int S = 0;    // global sink frames
  int Ss = 0;   // shot sink frames
  int W = 0;    // window frames
  int slots() const { return S + Ss + W; }
};

// Up to two slots of frame f in the shot that starts at fs; returns the count.
inline int slots_of(int64_t f, const Layout& L, int64_t fs, int out[2]) {
  if (f < L.S) {
    out[0] = int(f);
    return 1;
  }
  int n = 0;
  if (f >= fs && f < fs + L.Ss) out[n++] = L.S + int(f - fs);
  if (L.W > 0) out[n++] = L.S + L.Ss + int((f - L.S) % L.W);
  for (int j = 0; j < n; ++j) LL_CHECK(out[j] >= L.S && out[j] < L.slots());
  return n;
}

// Slots that hold frame f once f0 frames have been appended: its slots_of(), except
// that a ring slot has been reused by a later frame once f left the window.
inline int held_slots(int64_t f, int64_t f0, const Layout& L, int64_t fs, int out[2]) {
  int s[2];
  const int k = slots_of(f, L, fs, s);
  int n = 0;
  for (int j = 0; j < k; ++j)
    if (s[j] < L.S + L.Ss || f >= std::max<int64_t>(L.S, f0 - L.W)) out[n++] = s[j];
  return n;
}

// Single slot of frame f without a shot sink (-1 if dropped).
inline int64_t slot_of(int64_t f, int S, int W) {
  if (f < S) return f;
  if (W == 0) return -1;
  return S + (f - S) % W;
}

// The retained (cached, visible) frames of a chunk starting at f0, ascending: global
// sink, shot-sink frames no longer in the window, window oldest -> newest.
inline std::vector<int64_t> retained_frames(int64_t f0, const Layout& L, int64_t fs) {
  std::vector<int64_t> v;
  for (int64_t f = 0; f < std::min<int64_t>(L.S, f0); ++f) v.push_back(f);
  const int64_t wlo = std::max<int64_t>(L.S, f0 - L.W);
  for (int64_t f = std::max<int64_t>(L.S, fs); f < std::min<int64_t>({fs + L.Ss, f0, wlo}); ++f) v.push_back(f);
  for (int64_t f = wlo; f < f0; ++f) v.push_back(f);
  return v;
}
inline std::vector<int64_t> retained_frames(int64_t f0, int S, int W) { return retained_frames(f0, Layout{S, 0, W}, 0); }

// Number of cached frames a chunk starting at f0 sees.
inline int64_t cached_frames(int64_t f0, const Layout& L, int64_t fs) {
  const int64_t wlo = std::max<int64_t>(L.S, f0 - L.W);
  const int64_t shot = std::max<int64_t>(0, std::min<int64_t>({fs + L.Ss, f0, wlo}) - std::max<int64_t>(L.S, fs));
  return std::min<int64_t>(L.S, f0) + shot + (f0 - wlo > 0 ? f0 - wlo : 0);
}
inline int64_t cached_frames(int64_t f0, int S, int W) { return std::min<int64_t>(f0, int64_t(S) + W); }

// Slot runs holding the retained frames: (first slot, slot count), in slot order, at
// most three (adjacent runs merged).
struct SlotRun {
  int first, count;
};
inline std::vector<SlotRun> cache_runs(int64_t f0, const Layout& L, int64_t fs) {
  std::vector<SlotRun> runs;
  auto add = [&](int first, int count) {
    if (count <= 0) return;
    if (!runs.empty() && runs.back().first + runs.back().count == first) runs.back().count += count;
    else runs.push_back({first, count});
  };
  add(0, int(std::min<int64_t>(L.S, f0)));
  const int64_t wlo = std::max<int64_t>(L.S, f0 - L.W);
  const int64_t lo = std::max<int64_t>(L.S, fs), hi = std::min<int64_t>({fs + L.Ss, f0, wlo});
  if (hi > lo) add(L.S + int(lo - fs), int(hi - lo));
  add(L.S + L.Ss, int(std::max<int64_t>(0, f0 - wlo)));
  LL_CHECK(runs.size() <= 3);
  for (const SlotRun& r : runs) LL_CHECK(r.first >= 0 && r.count > 0 && r.first + r.count <= L.slots());
  return runs;
}

// Append n frames starting at f0 (shot start fs): for every slot that gets written, the
// LAST frame of the call that maps to it.  Entries come out in ascending slot order.
inline std::vector<WriteEntry> append_plan(int64_t f0, int n, const Layout& L, int64_t fs) {
  std::vector<int> last(size_t(L.slots()), -1);
  for (int i = 0; i < n; ++i) {
    int s[2];
    const int k = slots_of(f0 + i, L, fs, s);
    for (int j = 0; j < k; ++j) last[size_t(s[j])] = i;
  }
  std::vector<WriteEntry> out;
  for (int s = 0; s < L.slots(); ++s)
    if (last[size_t(s)] >= 0) out.push_back({last[size_t(s)], s, f0 + last[size_t(s)]});
  for (const WriteEntry& e : out) LL_CHECK(e.src >= 0 && e.src < n && e.slot >= 0 && e.slot < L.slots());
  return out;
}
inline std::vector<WriteEntry> append_plan(int64_t f0, int n, int S, int W) {
  return append_plan(f0, n, Layout{S, 0, W}, 0);
}

// Recache: block idx of the caller's tensor replaces retained frame idx in every slot
// that holds it.
inline std::vector<WriteEntry> recache_plan(int64_t f0, const Layout& L, int64_t fs) {
  std::vector<WriteEntry> out;
  const std::vector<int64_t> fr = retained_frames(f0, L, fs);
  for (size_t i = 0; i < fr.size(); ++i) {
    int s[2];
    const int k = held_slots(fr[i], f0, L, fs, s);
    for (int j = 0; j < k; ++j) out.push_back({int(i), s[j], fr[i]});
    LL_CHECK(k >= 1);   // every retained frame is held somewhere
  }
  LL_CHECK(int64_t(out.size()) <= L.slots());
  return out;
}
inline std::vector<WriteEntry> recache_plan(int64_t f0, int S, int W) { return recache_plan(f0, Layout{S, 0, W}, 0); }

// Window-only recache: block idx replaces window frame idx (oldest first) in every slot
// that holds it; the global sink and the shot frames outside the window are kept.
inline std::vector<WriteEntry> recache_window_plan(int64_t f0, const Layout& L, int64_t fs) {
  std::vector<WriteEntry> out;
  int idx = 0;
  for (int64_t f = std::max<int64_t>(L.S, f0 - L.W); f < f0; ++f, ++idx) {
    int s[2];
    const int k = held_slots(f, f0, L, fs, s);
    for (int j = 0; j < k; ++j) out.push_back({idx, s[j], f});
  }
  return out;
}
inline std::vector<WriteEntry> recache_window_plan(int64_t f0, int S, int W) {
  return recache_window_plan(f0, Layout{S, 0, W}, 0);
}

}  // namespace ll
