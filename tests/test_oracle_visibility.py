"""Pins for oracle.visibility and oracle.ring (CPU only).

Each check compares the oracle with something other than itself: a closed
form, a queue simulation of "keep the sink, evict the oldest", the page's
worked example, or the independent slot model.
"""

import os
from collections import deque

import pytest

from oracle import ring, visibility

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _queue_visible(f0, C, S, W):
    """Generate frames one at a time keeping sink frames forever and a FIFO
    of at most W other frames (the oldest leaves first)."""
    sink, fifo = [], deque()
    for f in range(f0):
        if f < S:
            sink.append(f)
        else:
            fifo.append(f)
            while len(fifo) > W:
                fifo.popleft()
    # frames below S may also be among the "last W" frames; the union counts them once
    last_w = set(range(max(0, f0 - W), f0))
    return sorted(set(sink) | set(fifo) | last_w | set(range(f0, f0 + C)))


@pytest.mark.parametrize("S", range(0, 5))
@pytest.mark.parametrize("W", [0, 1, 2, 3, 5, 6, 9, 12, 21, 25])
@pytest.mark.parametrize("C", [1, 2, 3, 4])
def test_visible_set_closed_form_and_queue(S, W, C):
    for f0 in range(0, 200, 1 if W < 10 else 3):
        v = visibility.visible_frames(f0, C, S, W)
        assert len(v) == min(f0, S + W) + C, (f0, C, S, W)
        assert v == _queue_visible(f0, C, S, W)
        # the own chunk is always visible, nothing later is
        assert all(f in v for f in range(f0, f0 + C))
        assert max(v) == f0 + C - 1 if v else True


@pytest.mark.parametrize("S", range(0, 5))
@pytest.mark.parametrize("W", [0, 1, 2, 5, 6, 12, 21])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 13, 30])
def test_ring_model_holds_exactly_the_cached_visible_set(S, W, n):
    if S + W == 0:
        pytest.skip("no slots")
    r = ring.RingModel(S, W)
    for _ in range(25):
        r.append(n)
        assert r.occupied_frames() == visibility.cached_visible_frames(r.f0, S, W)
        # one frame per slot, and every occupied slot is where slot_of puts it
        for s, f in enumerate(r.slot_frame):
            if f >= 0:
                assert r.slot_of(f) == s
        assert r.retained_frames() == visibility.cached_visible_frames(r.f0, S, W)


def test_ring_recache_rewrites_every_retained_slot():
    r = ring.RingModel(3, 12)
    for _ in range(10):
        r.append(3, src_of_frame=lambda f: ("append", f))
    frames = r.retained_frames()
    assert len(frames) == 15
    r.recache(15, src_of_block=lambda idx: ("recache", idx))
    for s, f in enumerate(r.slot_frame):
        assert r.slot_src[s][0] == "recache"
        assert frames[r.slot_src[s][1]] == f
    with pytest.raises(ValueError):
        r.recache(14)


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_golden_autoregressive_mask_example():
    # one latent frame per chunk z_i, no sink, window holding the whole history
    for q, vis, invis in _read_rows("ar_mask_example.txt"):
        q = int(q)
        v = visibility.visible_frames(q, 1, 0, 1000)
        assert v == [int(x) for x in vis.split(",")]
        for x in invis.split(","):
            assert int(x) not in v


def test_golden_attention_config_sink_and_window():
    ((C, W, S),) = [tuple(int(x) for x in r) for r in _read_rows("attention_config_example.txt")]
    for k in range(0, 60):
        f0 = k * C
        v = visibility.visible_frames(f0, C, S, W)
        if f0 >= S:
            # the first S frames stay visible however long the video gets
            assert all(f in v for f in range(S))
        # nothing older than the window is visible apart from the sink
        assert all(f < S or f >= f0 - W for f in v)
        # the context stops growing: at most S + W cached frames plus the chunk
        assert len(v) <= S + W + C


# ---- multi-shot sinks ------------------------------------------------------------

def _replay_shots(S, Ss, W, events):
    """Independent formulation by list slicing: events are ints (append a chunk of n
    frames, checking the visibility of that chunk first) or 'b' (a new shot starts).
    Yields (f0, n, fs, visible set of the chunk)."""
    video, since_shot, fs = [], [], 0
    for ev in events:
        if ev == "b":
            since_shot, fs = [], len(video)
            continue
        f0 = len(video)
        chunk = list(range(f0, f0 + ev))
        hist = set(video[:S]) | set(video[-W:] if W else []) | set(since_shot[:Ss])
        yield f0, ev, fs, hist | set(chunk)
        video += chunk
        since_shot += chunk


SHOT_EVENTS = [
    [3, 3, "b", 3, 3, 3, "b", 1, 1, 1, 1, 3, 3, 3, 3, 3],
    ["b", 2, 5, "b", "b", 1, 9, 2, "b", 4, 4, 4, 4],
    [1] * 5 + ["b"] + [1] * 20 + ["b"] + [7, 7, 7],
]


def test_shot_visibility_matches_independent_replay():
    for S in (0, 1, 3):
        for Ss in (0, 1, 3, 5):
            for W in (0, 2, 6, 12):
                for events in SHOT_EVENTS:
                    for f0, n, fs, want in _replay_shots(S, Ss, W, events):
                        got = visibility.visible_frames_shots(f0, n, S, Ss, W, fs)
                        assert got == sorted(want), (S, Ss, W, f0, fs)


def test_shot_visibility_reduces_to_sink_window():
    for f0 in range(0, 30):
        for S in (0, 2, 3):
            for W in (0, 4, 9):
                base = visibility.visible_frames(f0, 3, S, W)
                assert visibility.visible_frames_shots(f0, 3, S, 0, W, min(f0, 7)) == base
                # a shot sink inside the global sink adds nothing
                assert visibility.visible_frames_shots(f0, 3, S, min(S, f0), W, 0) == base


def test_ring_model_with_shots_holds_exactly_the_cached_visible_frames():
    for S in (0, 1, 3):
        for Ss in (1, 2, 4):
            for W in (0, 1, 5, 9):
                for events in SHOT_EVENTS:
                    r = ring.RingModel(S, W, Ss)
                    for ev in events:
                        if ev == "b":
                            r.begin_shot()
                            continue
                        r.append(ev)
                        want = visibility.cached_visible_frames(r.f0, S, W, Ss, r.fs)
                        assert r.occupied_frames() == want, (S, Ss, W, r.f0, r.fs)
                        assert r.retained_frames() == want
                        for s, f in enumerate(r.slot_frame):
                            if f >= 0:
                                assert s in r.slots_of(f)


def _fifo_window(f0, S, W):
    """The non-sink frames a FIFO of capacity W holds after frames 0 .. f0-1 arrive
    one at a time (sink frames never enter it), oldest first."""
    fifo = deque()
    for f in range(f0):
        if f >= S:
            fifo.append(f)
            while len(fifo) > W:
                fifo.popleft()
    return list(fifo)


@pytest.mark.parametrize("S", [0, 1, 3])
@pytest.mark.parametrize("W", [1, 2, 5, 12, 21])
@pytest.mark.parametrize("n", [1, 3, 4, 13])
def test_window_recache_rewrites_only_the_window(S, W, n):
    """techwalker.com article, §六: the narrower recache recomputes only the recent
    window and leaves the sink as it was.  Its frame list must equal a FIFO replay of
    the non-sink frames; sink slots keep their bytes, every window slot gets the block
    of its frame's position in that list."""
    r = ring.RingModel(S, W)
    for step in range(12):
        r.append(n, src_of_frame=lambda f: ("append", f))
        win = r.window_frames()
        assert win == _fifo_window(r.f0, S, W)
        assert win == [f for f in visibility.cached_visible_frames(r.f0, S, W) if f >= S]
        if not win:
            with pytest.raises(ValueError):
                r.recache_window(0)
            continue
        before = list(r.slot_src)
        r.recache_window(len(win), src_of_block=lambda idx: ("window", step, idx))
        for s, f in enumerate(r.slot_frame):
            if f < 0:
                continue
            if f < S:
                assert r.slot_src[s] == before[s] == ("append", f)
            else:
                assert r.slot_src[s] == ("window", step, win.index(f))
        with pytest.raises(ValueError):
            r.recache_window(len(win) + 1)
        # restore the appended bytes' tags so the next step's sink check stays exact
        for s, f in enumerate(r.slot_frame):
            if f >= 0:
                r.slot_src[s] = ("append", f)


def test_window_recache_with_shot_sink_keeps_shot_frames_outside_window():
    """With a shot sink, a shot-sink frame that has left the window is not part of the
    window recache; one still in the window is rewritten in both of its slots."""
    S, Ss, W = 1, 2, 3
    r = ring.RingModel(S, W, Ss)
    r.append(4, src_of_frame=lambda f: ("append", f))
    r.begin_shot()                          # shot starts at frame 4
    r.append(6, src_of_frame=lambda f: ("append", f))   # frames 4..9; window = 7, 8, 9
    assert r.window_frames() == [7, 8, 9]
    r.recache_window(3, src_of_block=lambda idx: ("window", idx))
    for s, f in enumerate(r.slot_frame):
        if f in (7, 8, 9):
            assert r.slot_src[s] == ("window", f - 7)
        elif f >= 0:
            assert r.slot_src[s] == ("append", f), (s, f)
    assert sorted(f for f in r.slot_frame if f >= 0) == [0, 4, 5, 7, 8, 9]
