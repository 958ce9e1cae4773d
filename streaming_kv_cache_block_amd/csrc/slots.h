// slots.h -- host-side slot arithmetic of the sink + window KV cache (header-only, C++17).
//
// Policy ("LongLive: Real-time Interactive Long Video Generation" explainer, dpshk.com,
// §五 and §六; techwalker.com LONGLIVE article, §六): a layer keeps the first S frames
// permanently (sink) and the K/V of the most recent W frames (window); anything older
// is evicted.  The library stores this in S + W fixed slots:
//
//   slot(f) = f                  for f < S          (sink slot, written once)
//           = S + (f - S) mod W  for f >= S, W > 0  (window ring)
//           = none               for f >= S, W = 0
//
// With f0 frames seen, the occupied slots are exactly [0, min(f0, S + W)): the sink
// slots fill first, then the ring fills S, S+1, ... before it wraps.  So the cached
// part of a chunk's context is one contiguous run of slots, scanned in physical
// order (softmax attention does not depend on the order of its keys).
//
// Builds with plain g++ (no HIP) for host-only tests.
#pragma once

#include <algorithm>
#include <cstdint>
#include <vector>

namespace ll {

struct WriteEntry {
  int src;   // frame index within the caller's tensor
  int slot;  // destination slot
  int64_t frame;  // absolute frame id stored in the slot
};

inline int64_t slot_of(int64_t f, int S, int W) {
  if (f < S) return f;
  if (W == 0) return -1;
  return S + (f - S) % W;
}

// Number of cached frames a chunk starting at f0 sees (= occupied slots).
inline int64_t cached_frames(int64_t f0, int S, int W) {
  return std::min<int64_t>(f0, int64_t(S) + W);
}

// Append n frames starting at f0: for every slot that gets written, the LAST frame of
// the call that maps to it.  Entries come out in ascending slot order.
inline std::vector<WriteEntry> append_plan(int64_t f0, int n, int S, int W) {
  std::vector<int> last(size_t(S) + W, -1);
  // Only the last S + W frames of a long call can survive; earlier ones are
  // overwritten within the call (or are sink frames, handled below).
  int first = 0;
  if (n > S + W) first = n - (S + W);
  for (int i = 0; i < n; ++i) {
    int64_t f = f0 + i;
    if (i < first && f >= S) continue;  // certainly replaced later in the call
    int64_t s = slot_of(f, S, W);
    if (s >= 0) last[size_t(s)] = i;
  }
  std::vector<WriteEntry> out;
  for (int s = 0; s < S + W; ++s)
    if (last[size_t(s)] >= 0) out.push_back({last[size_t(s)], s, f0 + last[size_t(s)]});
  return out;
}

// Logical order of the retained frames (sink ascending, then window oldest -> newest).
inline std::vector<int64_t> retained_frames(int64_t f0, int S, int W) {
  std::vector<int64_t> v;
  for (int64_t f = 0; f < std::min<int64_t>(S, f0); ++f) v.push_back(f);
  for (int64_t f = std::max<int64_t>(S, f0 - W); f < f0; ++f) v.push_back(f);
  return v;
}

// Recache: block idx of the caller's tensor replaces retained frame idx.
inline std::vector<WriteEntry> recache_plan(int64_t f0, int S, int W) {
  std::vector<WriteEntry> out;
  std::vector<int64_t> fr = retained_frames(f0, S, W);
  for (size_t i = 0; i < fr.size(); ++i)
    out.push_back({int(i), int(slot_of(fr[i], S, W)), fr[i]});
  return out;
}

// Window-only recache: block idx replaces window frame idx (oldest first); sink kept.
inline std::vector<WriteEntry> recache_window_plan(int64_t f0, int S, int W) {
  std::vector<WriteEntry> out;
  int idx = 0;
  for (int64_t f = std::max<int64_t>(S, f0 - W); f < f0; ++f, ++idx)
    out.push_back({idx, int(slot_of(f, S, W)), f});
  return out;
}

}  // namespace ll
