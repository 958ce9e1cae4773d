"""Host-side checks of the C ABI and the slot arithmetic (no GPU needed).

* the built library exports every function declared in include/ll_cache.h;
* invalid arguments are rejected with LL_ERR_INVALID / LL_ERR_STATE before any
  HIP call, and a missing device is reported as LL_ERR_HIP, never a crash;
* the library's slot arithmetic (slots.h, built with g++ and sanitizers) agrees
  bit-exactly with the oracle's independent slot model.
"""

import ctypes
import json
import os
import re
import subprocess

import pytest

import streaming_kv_cache_block_amd as ll
from streaming_kv_cache_block_amd import build as llbuild
from oracle import ring, visibility

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ll_cache.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ll_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ll.LIB_PATH):
        llbuild.build()
    return ll.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) == set(ll.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    D = ll.lib(debug=True)           # the debug build exports the same interface
    for n in names:
        assert hasattr(D, n), n


def test_create_rejects_invalid_arguments_before_touching_hip(L):
    h = ctypes.c_void_p()
    bad = [
        (0, 12, 128, 1560, 3, 12, 0),      # layers
        (1, 0, 128, 1560, 3, 12, 0),       # heads
        (1, 4097, 64, 16, 3, 12, 0),       # heads beyond the tile copies' 32-bit offsets
        (1, 12, 96, 1560, 3, 12, 0),       # head_dim
        (1, 12, 128, 0, 3, 12, 0),         # tokens per frame
        (1, 12, 128, 1560, -1, 12, 0),     # negative sink
        (1, 12, 128, 1560, 0, 0, 0),       # no slots
        (1, 12, 128, 1560, 64, 65, 0),     # too many slots
        (1, 12, 128, 1560, 3, 12, 5),      # dtype (0 bf16, 1 int8, 2 fp8, 3 mxfp4, 4 mxfp8)
        (1, 12, 128, 1560, 3, 12, -1),     # dtype
        (1, 1 << 20, 128, 1 << 20, 3, 12, 0),  # too large
    ]
    for args in bad:
        assert L.ll_cache_create(*args, ctypes.byref(h)) == ll.LL_ERR_INVALID, args
        assert L.ll_last_error()
        assert h.value is None
    assert L.ll_cache_create(1, 2, 64, 16, 3, 6, 0, None) == ll.LL_ERR_INVALID
    # shot sinks: S + Ss + W above the slot limit, a negative shot sink
    for args in [(1, 12, 128, 1560, 3, 3, 123, 0), (1, 12, 128, 1560, 3, -1, 12, 0)]:
        assert L.ll_cache_create_shots(*args, ctypes.byref(h)) == ll.LL_ERR_INVALID, args
        assert h.value is None


def test_calls_on_null_handle_are_invalid(L):
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    p16 = (p + 15) // 16 * 16
    assert L.ll_cache_append(None, 0, p16, p16, 1, None) == ll.LL_ERR_INVALID
    assert L.ll_attn_sink_window(None, 0, p16, p16, p16, 1, p16, None) == ll.LL_ERR_INVALID
    assert L.ll_attn_sink_window_noalloc(None, 0, p16, p16, p16, 1, p16, None) == ll.LL_ERR_INVALID
    assert L.ll_cache_recache(None, 0, p16, p16, 1, None) == ll.LL_ERR_INVALID
    assert L.ll_cache_recache_window(None, 0, p16, p16, 1, None) == ll.LL_ERR_INVALID
    assert L.ll_cache_recache_from_hidden(None, 0, p16, p16, p16, 1, 128, None) == ll.LL_ERR_INVALID
    f0 = ctypes.c_int64()
    assert L.ll_cache_frames_seen(None, 0, ctypes.byref(f0)) == ll.LL_ERR_INVALID
    L.ll_cache_destroy(None)


def test_projection_argument_checks(L):
    buf = ctypes.create_string_buffer(64)
    p16 = (ctypes.addressof(buf) + 15) // 16 * 16
    assert L.ll_kv_project(p16, p16, p16, 10, 96, 128, p16, p16, None) == ll.LL_ERR_INVALID   # d_in
    assert L.ll_kv_project(p16, p16, p16, 10, 128, 64, p16, p16, None) == ll.LL_ERR_INVALID   # d_out
    assert L.ll_kv_project(p16, p16, p16, 0, 128, 128, p16, p16, None) == ll.LL_ERR_INVALID   # n
    assert L.ll_kv_project(None, p16, p16, 10, 128, 128, p16, p16, None) == ll.LL_ERR_INVALID
    assert L.ll_kv_project(p16 + 2, p16, p16, 10, 128, 128, p16, p16, None) == ll.LL_ERR_INVALID  # alignment


def test_missing_device_is_reported_not_crashed(L):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    assert L.ll_cache_create(1, 2, 64, 16, 3, 6, 0, ctypes.byref(h)) == ll.LL_ERR_HIP
    assert b"hipGetDevice" in L.ll_last_error()


def test_python_binding_rejects_unknown_dtype():
    with pytest.raises(ValueError):
        ll.Cache(1, 2, 64, 16, 3, 6, kv_dtype="fp4")


def _run_cli(lines):
    cli = llbuild.SLOTS_CLI
    if not os.path.exists(cli):
        llbuild.build_slots_cli()
    r = subprocess.run([cli], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
    assert r.stderr == ""          # sanitizers print here
    return [json.loads(x) for x in r.stdout.splitlines()]


def _check_cli_against_model(lines, expect):
    got = _run_cli(lines)
    assert len(got) == len(expect)
    for g, (S, Ss, W, f0, fs, slot_frame, retained, window) in zip(got, expect):
        assert (g["S"], g["Ss"], g["W"], g["f0"], g["fs"]) == (S, Ss, W, f0, fs)
        assert g["slot_frame"] == slot_frame
        assert g["cached"] == len(retained)
        # the slot runs cover exactly the slots holding the retained frames, each frame once
        run_frames = [slot_frame[s] for first, count in g["runs"] for s in range(first, first + count)]
        assert sorted(run_frames) == retained
        # runs are in ascending slot order, disjoint and not adjacent (adjacent runs merge)
        for (a0, an), (b0, _) in zip(g["runs"], g["runs"][1:]):
            assert a0 + an < b0, g["runs"]
        assert len(g["runs"]) <= 3
        # recache: block idx -> the idx-th retained frame, in every slot the model holds it in
        blocks = {}
        for src, slot, frame in g["recache"]:
            assert slot_frame[slot] == frame
            blocks.setdefault(src, set()).add(frame)
        assert [blocks[i] for i in range(len(retained))] == [{f} for f in retained]
        held = sorted((s, f) for s, f in enumerate(slot_frame) if f >= 0)
        assert sorted((slot, frame) for _, slot, frame in g["recache"]) == held
        wb = {}
        for src, slot, frame in g["recache_window"]:
            assert slot_frame[slot] == frame
            wb.setdefault(src, set()).add(frame)
        assert [wb[i] for i in range(len(window))] == [{f} for f in window]


def test_slot_math_matches_oracle_ring_model():
    lines, expect = [], []
    for S in range(0, 5):
        for W in (0, 1, 2, 5, 6, 12, 21, 25):
            if S + W == 0:
                continue
            for pattern in ([3] * 30, [1] * 40, [4, 7, 2, 30, 1, 3, 50], [13, 13, 13]):
                lines.append(" ".join(map(str, [S, 0, W, *pattern])))
                r = ring.RingModel(S, W)
                for n in pattern:
                    r.append(n)
                    window = list(range(max(S, r.f0 - W), r.f0))
                    expect.append((S, 0, W, r.f0, r.fs, list(r.slot_frame), r.retained_frames(), window))
                    assert sorted(f for f in r.slot_frame if f >= 0) == visibility.cached_visible_frames(r.f0, S, W)
    _check_cli_against_model(lines, expect)


def test_slot_math_with_shot_sinks_matches_oracle_ring_model():
    lines, expect = [], []
    patterns = [[3, 3, "b", 3, 3, 3, "b", 1, 1, 1, 3, 3, 3, 3],
                ["b", 2, 5, "b", "b", 1, 9, 2, "b", 4, 4, 4, 4, 30, "b", 3],
                [1] * 5 + ["b"] + [1] * 20 + ["b"] + [7, 7, 7]]
    for S in (0, 1, 3):
        for Ss in (1, 2, 3, 6):
            for W in (0, 1, 5, 12):
                for pattern in patterns:
                    lines.append(" ".join(map(str, [S, Ss, W, *pattern])))
                    r = ring.RingModel(S, W, Ss)
                    for ev in pattern:
                        if ev == "b":
                            r.begin_shot()
                            continue
                        r.append(ev)
                        window = list(range(max(S, r.f0 - W), r.f0))
                        expect.append((S, Ss, W, r.f0, r.fs, list(r.slot_frame), r.retained_frames(), window))
    _check_cli_against_model(lines, expect)


def _check_split_plan(rec):
    B, J, n_cu = rec["B"], rec["J"], rec["n_cu"]
    by_blk = {}
    for wg, blk, ja, jb, npc, slot, tail0 in rec["pieces"]:
        assert 0 <= wg < (n_cu if rec["on"] else (B + 7) // 8 * 8)
        assert 0 <= blk < B and 0 <= ja < jb <= J
        by_blk.setdefault(blk, []).append((ja, jb, npc, slot, tail0))
    assert sorted(by_blk) == list(range(B)), "every block runs"
    used = set()
    for blk, ps in by_blk.items():
        ps.sort()
        # the pieces tile the block's key walk [0, J) exactly once
        assert ps[0][0] == 0 and ps[-1][1] == J
        assert all(a[1] == b[0] for a, b in zip(ps, ps[1:]))
        assert all(p[2] == len(ps) for p in ps) and len(ps) <= 3
        if len(ps) == 1:
            continue
        assert rec["on"]
        assert ps[0][3] == blk                                    # head piece: the block's own slot
        t0 = {p[4] for p in ps}
        assert len(t0) == 1
        tails = [p[3] for p in ps[1:]]
        assert tails == [ps[0][4] + k for k in range(len(tails))]  # tail slots tail0, tail0 + 1
        for s in [blk] + tails:
            assert 0 <= s < rec["slots"] and s not in used, (blk, s)
            used.add(s)


def test_split_walk_plan_covers_every_key_once_with_unique_slots():
    """The split attention launch's plan (split_plan.h, g++ build): each block's key
    tiles are walked exactly once across its pieces, at most three pieces per block,
    and every partial result has its own slot below the work area's 2 x CUs."""
    lines = []
    for n_cu in (256, 304, 80, 8):
        for B in (1, 7, 8, 9, 24, 100, 152, 156, 168, 200, 208, 228, 255, 256, 300):
            for J in (1, 31, 32, 33, 64, 100, 440, 659, 2000):
                lines.append(f"split {B} {J} {n_cu}")
    recs = _run_cli(lines)
    assert len(recs) == len(lines)
    n_on = 0
    for rec in recs:
        _check_split_plan(rec)
        n_on += rec["on"]
        if rec["B"] == 228 and rec["J"] == 440 and rec["n_cu"] == 256:
            assert rec["on"] == 1     # the steady shape takes the split walk
    assert n_on > 50


class _FakeTensor:
    """Stands in for a device tensor in the binding's argument checks (no GPU here):
    shape and element count only; the checks must fire before any pointer is taken."""

    def __init__(self, *shape):
        self.shape = shape

    def numel(self):
        n = 1
        for d in self.shape:
            n *= d
        return n


def test_binding_rejects_mis_shaped_tensors_before_the_library():
    c = ll.Cache.__new__(ll.Cache)          # a handle-less object: only the checks run
    c.layers, c.heads, c.head_dim, c.T, c.S, c.W, c.Ss = 1, 12, 128, 1560, 3, 12, 0
    good = _FakeTensor(3 * 1560, 12, 128)
    for bad in (_FakeTensor(3 * 1560, 12, 64), _FakeTensor(3 * 1560, 8, 128), _FakeTensor(2 * 1560 + 1, 12, 128)):
        with pytest.raises(ValueError):
            c.attn(0, good, good, bad, out=good)
        with pytest.raises(ValueError):
            c.attn(0, good, good, good, out=bad)
        with pytest.raises(ValueError):
            c.append(0, good, bad)
        with pytest.raises(ValueError):
            c.recache(0, good, bad)
    with pytest.raises(ValueError):           # explicit n_frames larger than the tensors
        c.attn(0, good, good, good, out=good, n_frames=4)
    with pytest.raises(ValueError):
        c.recache_from_hidden(0, _FakeTensor(15 * 1560, 1536), _FakeTensor(1536, 1536), _FakeTensor(1536, 1024))
    with pytest.raises(ValueError):
        ll.kv_project(_FakeTensor(100, 1536), _FakeTensor(1536, 1536), _FakeTensor(1536, 1535))
