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

``recache_window(n)`` is the narrower recache of the techwalker.com article,
§六 (recomputation limited to the most recent window, the sink tokens kept as
they are).  Its logical list is the window frames alone, [max(S, f0 - W), f0)
oldest to newest, and n must equal its length (at least 1); block idx replaces
frame list[idx] in every slot that holds it.  Sink slots (and, with a shot
sink, shot-sink frames that have left the window) keep their bytes; f0 is
unchanged.

Each slot records which frame it holds (``slot_frame``, -1 = empty) and a
caller-defined token for where its bytes came from (``slot_src``), so tests
can compare GPU slot bytes with the bytes of the frame the model says are
there.

Shot sinks (LongLive-2.0 explainer, wmrh.cn, §16; reading in visibility.py):
with Ss > 0 the layer has S + Ss + W slots: [0, S) global sink, [S, S + Ss)
shot sink, [S + Ss, S + Ss + W) window ring.  A frame f >= S of the current
shot's first Ss frames (fs <= f < fs + Ss) is written to its shot slot
S + (f - fs) AND to its ring slot S + Ss + (f - S) mod W; ``begin_shot()``
sets fs = f0 and empties the shot slots.  The frames held are then exactly
the cached part of V(f0; fs); a frame held twice is one frame.  Recache
takes the retained frames in ascending order and writes block idx to every
slot holding frame idx.
"""


class RingModel:
    def __init__(self, S: int, W: int, Ss: int = 0):
        if S < 0 or W < 0 or Ss < 0 or S + Ss + W == 0:
            raise ValueError("need S, Ss, W >= 0 and S + Ss + W > 0")
        self.S, self.W, self.Ss = S, W, Ss
        self.f0 = 0
        self.fs = 0
        self.slot_frame = [-1] * (S + Ss + W)
        self.slot_src = [None] * (S + Ss + W)

    def slots_of(self, f: int) -> list:
        """Slots that store frame f (given the current shot)."""
        if f < self.S:
            return [f]
        out = []
        if self.fs <= f < self.fs + self.Ss:
            out.append(self.S + (f - self.fs))
        if self.W > 0:
            out.append(self.S + self.Ss + (f - self.S) % self.W)
        return out

    def slot_of(self, f: int):
        """The single slot of frame f when there is no shot sink (None if dropped)."""
        s = self.slots_of(f)
        if self.Ss:
            raise ValueError("slot_of: frames may have two slots with a shot sink")
        return s[0] if s else None

    def begin_shot(self):
        self.fs = self.f0
        for s in range(self.S, self.S + self.Ss):
            self.slot_frame[s] = -1
            self.slot_src[s] = None

    def append(self, n: int, src_of_frame=lambda f: f):
        if n <= 0:
            raise ValueError("append needs n > 0")
        for i in range(n):
            f = self.f0 + i
            for s in self.slots_of(f):
                self.slot_frame[s] = f
                self.slot_src[s] = src_of_frame(f)
        self.f0 += n

    def retained_frames(self) -> list:
        """Logical recache order: the cached visible frames ascending (sink, shot sink,
        then window oldest -> newest)."""
        sink = set(range(0, min(self.S, self.f0)))
        shot = set(range(max(self.S, self.fs), min(self.fs + self.Ss, self.f0)))
        window = set(range(max(self.S, self.f0 - self.W), self.f0))
        return sorted(sink | shot | window)

    def recache(self, n: int, src_of_block=lambda idx: idx):
        frames = self.retained_frames()
        if n != len(frames):
            raise ValueError("recache: n must equal the number of retained frames")
        for idx, f in enumerate(frames):
            held = [s for s, g in enumerate(self.slot_frame) if g == f]
            if not held:
                raise AssertionError("ring model inconsistent")
            for s in held:
                self.slot_src[s] = src_of_block(idx)

    def window_frames(self) -> list:
        """Logical order of the window-only recache: the non-sink frames of the most
        recent window, oldest -> newest."""
        return list(range(max(self.S, self.f0 - self.W), self.f0))

    def recache_window(self, n: int, src_of_block=lambda idx: idx):
        frames = self.window_frames()
        if n != len(frames) or n == 0:
            raise ValueError("recache_window: n must equal the number of window frames (>= 1)")
        for idx, f in enumerate(frames):
            held = [s for s, g in enumerate(self.slot_frame) if g == f]
            if not held:
                raise AssertionError("ring model inconsistent")
            for s in held:
                self.slot_src[s] = src_of_block(idx)

    def occupied_frames(self) -> list:
        return sorted(set(f for f in self.slot_frame if f >= 0))
