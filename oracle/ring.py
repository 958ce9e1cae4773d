"""Independent model of the fixed-capacity per-layer slot store (test infrastructure only).

Sources
-------
* dpshk.com explainer of "LongLive: Real-time Interactive Long Video
  Generation", §二 (after a chunk is generated its K/V enter the cache),
  §五 (K/V older than the window are evicted), §六 (the sink frames' K/V stay
  permanently), §三 item 5 (recache: drop the old cache, keep the latents,
  recompute a fresh cache under the new prompt and use it instead).
* techwalker.com article on LONGLIVE, §六 (old cache entries are retired as
  new ones arrive so memory stays bounded).

Storage model (the library's layout, stated here independently of it)
-------------------------------------------------------------------
A layer owns S + W slots.  Frame f lives in

    slot(f) = f                      if f < S        (sink, permanent)
            = S + (f - S) mod W      if f >= S, W > 0 (window ring)
            = none (dropped)         if f >= S, W = 0

``append(n)`` writes frames f0 .. f0+n-1 in that order (a later frame that
maps to the same slot replaces an earlier one), then f0 += n.

``recache(n)`` requires n = min(f0, S + W).  Its logical frame list is the
sink frames [0, min(S, f0)) in ascending order followed by the window frames
[max(S, f0 - W), f0) oldest to newest; block idx of the recache tensors
replaces frame list[idx] in slot(list[idx]).  f0 is unchanged.

Each slot records which frame it holds (``slot_frame``, -1 = empty) and a
caller-defined token for where its bytes came from (``slot_src``), so tests
can compare GPU slot bytes with the bytes of the frame the model says are
there.
"""


class RingModel:
    def __init__(self, S: int, W: int):
        if S < 0 or W < 0 or S + W == 0:
            raise ValueError("need S >= 0, W >= 0, S + W > 0")
        self.S, self.W = S, W
        self.f0 = 0
        self.slot_frame = [-1] * (S + W)
        self.slot_src = [None] * (S + W)

    def slot_of(self, f: int):
        if f < self.S:
            return f
        if self.W == 0:
            return None
        return self.S + (f - self.S) % self.W

    def append(self, n: int, src_of_frame=lambda f: f):
        if n <= 0:
            raise ValueError("append needs n > 0")
        for i in range(n):
            f = self.f0 + i
            s = self.slot_of(f)
            if s is None:
                continue
            self.slot_frame[s] = f
            self.slot_src[s] = src_of_frame(f)
        self.f0 += n

    def retained_frames(self) -> list:
        """Logical recache order: sink ascending, then window oldest -> newest."""
        sink = list(range(0, min(self.S, self.f0)))
        window = list(range(max(self.S, self.f0 - self.W), self.f0))
        return sink + window

    def recache(self, n: int, src_of_block=lambda idx: idx):
        frames = self.retained_frames()
        if n != len(frames) or n != min(self.f0, self.S + self.W):
            raise ValueError("recache: n must equal min(f0, S + W)")
        for idx, f in enumerate(frames):
            s = self.slot_of(f)
            if self.slot_frame[s] != f:
                raise AssertionError("ring model inconsistent")
            self.slot_src[s] = src_of_block(idx)

    def occupied_frames(self) -> list:
        return sorted(f for f in self.slot_frame if f >= 0)
