"""GPU parity on seeded random cache configurations.

24 configurations drawn from a fixed seed: sink 0-4, window 0-10, shot sink 0-2 frames,
16 / 48 / 96 tokens per frame, 1-3 heads, head_dim 64 or 128, chunks of 1-3 frames with
ragged lengths, bf16 / int8 / fp8 caches; and 12 more from another seed with MXFP4 / MXFP8
caches.  Each runs 10 chunks with a shot start (when
the cache has a shot sink), a full recache after chunk 5 and a window-only recache after
chunk 7 (when the cache holds such frames).  Every attention output is compared with the
oracle in full; the slot maps and bytes are compared after every recache and at the end.
The hand-picked GPU tests cover the workloads' shapes and the known edge cases; these
cover combinations of them that no one picked.
"""

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from oracle import attention

from helpers import History, check_slots, compare_attention

pytestmark = pytest.mark.gpu


def _configs(n=24, seed=790, formats=("bf16", "int8", "fp8"), first=0):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        S, W, Ss = int(rng.integers(0, 5)), int(rng.integers(0, 11)), int(rng.choice([0, 0, 1, 2]))
        if S + W + Ss == 0:
            continue
        T = int(rng.choice([16, 48, 96]))
        H = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128]))
        C = int(rng.integers(1, 4))
        kv = str(rng.choice(list(formats)))
        out.append((first + len(out), S, W, Ss, T, H, D, C, kv))
    return out


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()
    return torch


@pytest.mark.parametrize("cfg", _configs() + _configs(12, 791, ("mxfp4", "mxfp8"), first=24),
                         ids=lambda c: "i%d_S%d_W%d_Ss%d_T%d_H%d_D%d_C%d_%s" % c)
def test_random_configuration(torch_gpu, cfg):
    i, S, W, Ss, T, H, D, C, kv = cfg
    rng = np.random.default_rng(800 + i)
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv, shot_sink=Ss)
    hist = History(S, W, T, Ss)
    shot_at = int(rng.integers(2, 6)) if Ss else -1
    for k in range(10):
        what = f"config {cfg} chunk {k} f0 {hist.f0}"
        print(what, flush=True)
        if k == shot_at:
            cache.begin_shot(0)
            hist.begin_shot()
        n = int(rng.integers(1, C + 1))   # ragged chunk lengths
        shape = (n * T, H, D)
        q, kc, vc = (synth.normal_bf16(shape, 1.0, 801, i, k, t) for t in range(3))
        out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
        ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, kv=kv, shot=hist.shot)
        compare_attention(out, ref, what)
        cache.append(0, synth.to_device(kc), synth.to_device(vc))
        hist.append(kc, vc)
        if k == 5:
            m = len(hist.model.retained_frames())
            K_all, V_all = (synth.normal_bf16((m * T, H, D), 1.0, 802, i, t) for t in range(2))
            cache.recache(0, synth.to_device(K_all), synth.to_device(V_all))
            hist.recache(K_all, V_all)
            check_slots(cache, 0, hist, kv=kv)
        if k == 7 and hist.model.window_frames():
            m = len(hist.model.window_frames())
            K_w, V_w = (synth.normal_bf16((m * T, H, D), 1.0, 803, i, t) for t in range(2))
            cache.recache_window(0, synth.to_device(K_w), synth.to_device(V_w))
            hist.recache_window(K_w, V_w)
            check_slots(cache, 0, hist, kv=kv)
    check_slots(cache, 0, hist, kv=kv)
    cache.close()
