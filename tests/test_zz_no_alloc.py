"""The allocation-free attention entry point against the ordinary one, through the C ABI.

ll_attn_sink_window_noalloc runs the same kernels with the library's static per-GPU
scratch in place of the layer's work area.  Two calls in a row, the second with a
smaller input, must give exactly the bytes of ll_attn_sink_window on the same inputs
(the merge order of the split walk is fixed); the scratch keeps the first call's
contents, so the second also shows its counters were left at zero.  A small chunk that
does not split the walk uses no scratch.  Device memory in use must not grow.
"""

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from oracle import attention

from helpers import History, compare_attention, sample_rows

pytestmark = pytest.mark.gpu

T, H, D, S, W, C = 1560, 12, 128, 3, 12, 3


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()
    return torch


def test_noalloc_attention_matches_the_allocating_entry_point(torch_gpu):
    torch = torch_gpu
    shape = (C * T, H, D)
    cache = ll.Cache(1, H, D, T, S, W)
    hist = History(S, W, T)
    for k in range(6):
        kb, vb = (synth.normal_bf16(shape, 0.5, 760, t, k) for t in range(2))
        cache.append(0, synth.to_device(kb), synth.to_device(vb))
        hist.append(kb, vb)
    torch.cuda.synchronize()
    for n_frames, tag in ((3, "full chunk (split walk)"), (2, "smaller chunk (split walk)"),
                          (1, "one frame (split walk)")):
        nq = n_frames * T
        q, kc, vc = (synth.normal_bf16((nq, H, D), 0.5, 761, n_frames, t) for t in range(3))
        qd, kd, vd = (synth.to_device(x) for x in (q, kc, vc))
        want = cache.attn(0, qd, kd, vd)
        got = torch.empty_like(want)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        cache.attn_noalloc(0, qd, kd, vd, got)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] >= free0, "device memory in use grew"
        print(f"noalloc {tag}: nq={nq}", flush=True)
        assert np.array_equal(synth.to_bits(got), synth.to_bits(want)), tag
        rows = sample_rows(nq, T, seed=762 + n_frames, n_random=16)
        ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, rows=rows)
        compare_attention(synth.to_bits(got)[rows], ref, tag, scale_gate=True)
    cache.close()


def test_noalloc_attention_without_split_and_low_bit_cache(torch_gpu):
    """A toy-sized chunk (no split, no scratch) and an int8 cache at full shape (split,
    scaled tiles), each equal to the allocating entry point."""
    torch = torch_gpu
    small = ll.Cache(1, 2, 64, 16, 3, 6)
    for k in range(4):
        small.append(0, *(synth.to_device(synth.normal_bf16((48, 2, 64), 1.0, 763, t, k)) for t in range(2)))
    q, kc, vc = (synth.to_device(synth.normal_bf16((48, 2, 64), 1.0, 764, t)) for t in range(3))
    want = small.attn(0, q, kc, vc)
    got = small.attn_noalloc(0, q, kc, vc, torch.empty_like(want))
    assert np.array_equal(synth.to_bits(got), synth.to_bits(want))
    small.close()
    big = ll.Cache(1, H, D, T, S, 21, kv_dtype="int8")
    shape = (C * T, H, D)
    for k in range(9):
        big.append(0, *(synth.to_device(synth.normal_bf16(shape, 0.5, 765, t, k)) for t in range(2)))
    q, kc, vc = (synth.to_device(synth.normal_bf16(shape, 0.5, 766, t)) for t in range(3))
    want = big.attn(0, q, kc, vc)
    for _ in range(2):
        got = big.attn_noalloc(0, q, kc, vc, torch.empty_like(want))
        assert np.array_equal(synth.to_bits(got), synth.to_bits(want))
    big.close()
