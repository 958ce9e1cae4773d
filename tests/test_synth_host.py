"""Pins for the seeded input generator (synth.philox) and its device twin's library (CPU).

The generator is input preparation, shared by both sides; these checks tie it to its
published definition so that a device draw regenerated on the host means the same thing.
"""

import ctypes
import os
import statistics

import numpy as np
import pytest

import synth
from synth import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answer_vectors():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        ctr = [int(x, 16) for x in r[0:4]]
        key = [int(x, 16) for x in r[4:6]]
        want = [int(x, 16) for x in r[6:10]]
        got = philox.philox4x32_10(*[np.array([c], dtype=np.uint32) for c in ctr], *key)
        assert [int(g[0]) for g in got] == want


def test_element_i_takes_word_i_mod_4_of_block_i_div_4():
    key = synth.key64(1, 2, 3)
    w = philox.words(11, key)
    for i in range(11):
        b = i // 4
        out = philox.philox4x32_10(np.array([b], np.uint32), np.array([0], np.uint32), 0, 0,
                                   key & 0xFFFFFFFF, key >> 32)
        assert w[i] == out[i % 4][0]
    # a block index past 2^32 carries into counter word 1
    big = philox.philox4x32_10(np.array([5], np.uint32), np.array([1], np.uint32), 0, 0, 7, 9)
    assert big[0][0] != philox.philox4x32_10(np.array([5], np.uint32), np.array([0], np.uint32), 0, 0, 7, 9)[0][0]


def test_quantile_table_matches_an_independent_inverse_cdf():
    t = philox.normal_table()
    assert t.dtype == np.float32 and t.shape == (65536,)
    assert (np.diff(t) > 0).all()                       # strictly increasing
    assert np.array_equal(t, -t[::-1])                  # symmetric about zero
    nd = statistics.NormalDist()
    for j in list(range(0, 65536, 4099)) + [0, 1, 32767, 32768, 65534, 65535]:
        want = nd.inv_cdf((j + 0.5) / 65536)
        assert abs(float(t[j]) - want) <= 2e-7 * max(1.0, abs(want)), j


def test_draws_are_bf16_rounded_scaled_quantiles_with_the_right_moments():
    key = synth.key64(4, 5)
    x = synth.normal_bf16_philox((200_000,), 0.5, 4, 5)
    j = philox.words(200_000, key) >> np.uint32(16)
    vals = philox.normal_table()[j] * np.float32(0.5)
    assert np.array_equal(x, synth.f32_to_bf16_bits(vals))
    f = synth.bf16_bits_to_f32(x).astype(np.float64)
    assert abs(f.mean()) < 0.005 and abs(f.std() - 0.5) < 0.005
    # different keys give different streams; the same key the same
    assert not np.array_equal(x[:64], synth.normal_bf16_philox((64,), 0.5, 4, 6))
    assert np.array_equal(x[:64], synth.normal_bf16_philox((64,), 0.5, 4, 5))


def test_device_twin_library_exports_its_fill():
    from synth import device
    from streaming_kv_cache_block_amd import build as llbuild
    if not os.path.exists(device.LIB_PATH):
        llbuild.build()
    L = ctypes.CDLL(device.LIB_PATH)
    assert hasattr(L, "synth_fill_normal_bf16")
