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


def test_create_rejects_invalid_arguments_before_touching_hip(L):
    h = ctypes.c_void_p()
    bad = [
        (0, 12, 128, 1560, 3, 12, 0),      # layers
        (1, 0, 128, 1560, 3, 12, 0),       # heads
        (1, 12, 96, 1560, 3, 12, 0),       # head_dim
        (1, 12, 128, 0, 3, 12, 0),         # tokens per frame
        (1, 12, 128, 1560, -1, 12, 0),     # negative sink
        (1, 12, 128, 1560, 0, 0, 0),       # no slots
        (1, 12, 128, 1560, 64, 65, 0),     # too many slots
        (1, 12, 128, 1560, 3, 12, 3),      # dtype
        (1, 1 << 20, 128, 1 << 20, 3, 12, 0),  # too large
    ]
    for args in bad:
        assert L.ll_cache_create(*args, ctypes.byref(h)) == ll.LL_ERR_INVALID, args
        assert L.ll_last_error()
        assert h.value is None
    assert L.ll_cache_create(1, 2, 64, 16, 3, 6, 0, None) == ll.LL_ERR_INVALID


def test_calls_on_null_handle_are_invalid(L):
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    p16 = (p + 15) // 16 * 16
    assert L.ll_cache_append(None, 0, p16, p16, 1, None) == ll.LL_ERR_INVALID
    assert L.ll_attn_sink_window(None, 0, p16, p16, p16, 1, p16, None) == ll.LL_ERR_INVALID
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


def test_slot_math_matches_oracle_ring_model():
    lines, expect = [], []
    for S in range(0, 5):
        for W in (0, 1, 2, 5, 6, 12, 21, 25):
            if S + W == 0:
                continue
            for pattern in ([3] * 30, [1] * 40, [4, 7, 2, 30, 1, 3, 50], [13, 13, 13]):
                lines.append(" ".join(map(str, [S, W, *pattern])))
                r = ring.RingModel(S, W)
                for n in pattern:
                    r.append(n)
                    expect.append((S, W, r.f0, list(r.slot_frame), r.retained_frames()))
    got = _run_cli(lines)
    assert len(got) == len(expect)
    for g, (S, W, f0, slot_frame, retained) in zip(got, expect):
        assert (g["S"], g["W"], g["f0"]) == (S, W, f0)
        assert g["slot_frame"] == slot_frame
        # recache: block idx -> the idx-th retained frame, in the slot the model holds it
        assert [e[2] for e in g["recache"]] == retained
        assert [e[0] for e in g["recache"]] == list(range(len(retained)))
        for src, slot, frame in g["recache"]:
            assert slot_frame[slot] == frame
        window = [f for f in retained if f >= S]
        assert [e[2] for e in g["recache_window"]] == window
        assert sorted(f for f in g["slot_frame"] if f >= 0) == visibility.cached_visible_frames(f0, S, W)
