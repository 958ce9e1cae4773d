"""Which latent frames a chunk may attend to (test infrastructure only).

Sources
-------
* dpshk.com explainer of "LongLive: Real-time Interactive Long Video
  Generation", §五 (short window: only the most recent history is looked at,
  older K/V are evicted) and §六 (frame sink: the first frames stay in the KV
  cache permanently; the cache is the sink frames' K/V plus the recent
  window's K/V).
* techwalker.com article "英伟达突破视频生成瓶颈：LONGLIVE…", §六: a chunk is
  3 latent frames, the local window is 9 latent frames, the first 3 latent
  frames are the globally visible sink.
* wmrh.cn explainer of LongLive-2.0, §6: a chunk sees the earlier chunks and
  itself, never a later chunk (noisy z2 sees z0, z1 and its own z2, not z3).

Reading adopted where the pages are silent
------------------------------------------
* The window counts cached (already finished) frames only; the chunk being
  generated is a third, separate part of the context.
* Sink and window are combined as a set union: a frame counts once.
* Inside its own chunk every query sees every key (the block of the
  block-causal mask is the chunk).

The visible set of a chunk that starts at frame ``f0`` and spans ``C``
frames is

    V(f0) = {f : 0 <= f < min(S, f0)}
          U {f : max(0, f0 - W) <= f < f0}
          U {f0, ..., f0 + C - 1}.

Multi-shot sinks (LongLive-2.0 explainer, wmrh.cn, §16): a global sink that every
shot attends to and a shot sink that keeps the current shot's own early context.
Reading adopted (the page names the two levels only): the global sink is the
first S frames of the video as above; the shot sink is the first Ss frames of
the current shot, which starts at frame fs (fs <= f0); a chunk sees their union
with the window and its own chunk:

    V(f0; fs) = V(f0) U {f : fs <= f < min(fs + Ss, f0)}.

With Ss = 0 (or a shot sink inside the global sink) this is V(f0).

This module never refers to slots, rings or physical positions.
"""

import numpy as np


def visible_frames(f0: int, C: int, S: int, W: int) -> list:
    """Sorted list of the frames visible to the chunk [f0, f0+C)."""
    if f0 < 0 or C < 0 or S < 0 or W < 0:
        raise ValueError("negative argument")
    sink = set(range(0, min(S, f0)))
    window = set(range(max(0, f0 - W), f0))
    own = set(range(f0, f0 + C))
    return sorted(sink | window | own)


def visible_frames_shots(f0: int, C: int, S: int, Ss: int, W: int, fs: int) -> list:
    """Sorted frames visible to the chunk [f0, f0+C) in the shot that starts at fs."""
    if Ss < 0 or fs < 0 or fs > f0:
        raise ValueError("need Ss >= 0 and 0 <= fs <= f0")
    shot = set(range(fs, min(fs + Ss, f0)))
    return sorted(set(visible_frames(f0, C, S, W)) | shot)


def cached_visible_frames(f0: int, S: int, W: int, Ss: int = 0, fs: int = 0) -> list:
    """The history part of V(f0) (with a shot sink of Ss frames from fs, if any)."""
    return visible_frames_shots(f0, 0, S, Ss, W, fs)


def frame_mask(f0: int, C: int, S: int, W: int, n_frames: int, Ss: int = 0, fs: int = 0) -> np.ndarray:
    """Boolean mask over frames [0, n_frames): True where the frame is in V(f0; fs)."""
    m = np.zeros(n_frames, dtype=bool)
    for f in visible_frames_shots(f0, C, S, Ss, W, fs):
        if f < n_frames:
            m[f] = True
    return m


def key_mask(f0: int, C: int, S: int, W: int, frame_of_key: np.ndarray) -> np.ndarray:
    """Boolean mask over keys: key j is visible iff frame_of_key[j] is in V(f0)."""
    vis = np.zeros(int(frame_of_key.max()) + 1 if frame_of_key.size else 0, dtype=bool)
    for f in visible_frames(f0, C, S, W):
        if f < vis.size:
            vis[f] = True
    return vis[frame_of_key] if frame_of_key.size else np.zeros(0, dtype=bool)
