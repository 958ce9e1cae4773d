"""GPU parity of the multi-shot cache: a global sink, a shot sink and the window.

Reading tested (LongLive-2.0 explainer, wmrh.cn, §16; oracle.visibility): a chunk
starting at f0 in the shot that started at fs sees the first S frames of the video,
the first Ss frames of its shot, the last W frames and its own chunk.  Slot contents
are compared bit for bit with the oracle's slot model after every call (a shot-sink
frame still in the window is held in two slots), attention with the oracle fed the
same visible set, and the frame-id probe checks the visible set structurally.
Inputs: bf16 N(0, 1) draws from fixed seeds.
"""

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from oracle import attention, bf16, visibility

from helpers import History, check_slots, compare_attention, sample_rows

pytestmark = pytest.mark.gpu

EVENTS = [3, 3, "b", 3, 3, 3, 3, "b", 1, 1, 3, "b", "b", 3, 3, 3, 3, 3, 3]


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()
    return torch


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S,Ss,W", [(3, 3, 6), (0, 2, 4), (2, 5, 3), (1, 4, 0), (3, 1, 9)])
def test_shot_frame_id_probe(torch_gpu, D, S, Ss, W):
    """K = 0 and V one-hot at d = frame id mod D: out[d] = (#visible tokens of frame d) /
    (#visible tokens), which names exactly the frames the kernel read."""
    torch = torch_gpu
    T, H = 40, 3
    cache = ll.Cache(1, H, D, T, S, W, shot_sink=Ss)
    f0, fs = 0, 0
    for ev in EVENTS:
        if ev == "b":
            cache.begin_shot(0)
            fs = f0
            continue
        n = ev
        q = torch.randn((n * T, H, D), device="cuda").to(torch.bfloat16)
        kz = torch.zeros((n * T, H, D), device="cuda", dtype=torch.bfloat16)
        v = torch.zeros((n * T, H, D), device="cuda", dtype=torch.bfloat16)
        for i in range(n):
            v[i * T:(i + 1) * T, :, (f0 + i) % D] = 1.0
        out = cache.attn(0, q, kz, v)
        vis = visibility.visible_frames_shots(f0, n, S, Ss, W, fs)
        expect = np.zeros(D)
        for f in vis:
            expect[f % D] += T
        expect /= len(vis) * T
        got = bf16.to_f32(synth.to_bits(out)).astype(np.float64)
        want = bf16.to_f32(bf16.round_f32(expect.astype(np.float32))).astype(np.float64)
        assert np.abs(got - want[None, None, :]).max() <= np.abs(want).max() * 2 ** -7, (f0, fs, n)
        cache.append(0, kz, v)
        assert cache.shot_start(0) == fs
        f0 += n


def _rollout(torch, S, Ss, W, T, H, D, kv, seed, recache_at=(), fused_recache_at=()):
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv, shot_sink=Ss)
    hist = History(S, W, T, Ss)
    step = 0
    for ev in EVENTS:
        if ev == "b":
            cache.begin_shot(0)
            hist.begin_shot()
            check_slots(cache, 0, hist, kv=kv)
            continue
        n = ev
        shape = (n * T, H, D)
        if step in recache_at or step in fused_recache_at:
            m = len(hist.model.retained_frames())
            if step in recache_at:
                K_all = synth.normal_bf16((m * T, H, D), 1.0, seed, 50, step, 0)
                V_all = synth.normal_bf16((m * T, H, D), 1.0, seed, 50, step, 1)
                cache.recache(0, synth.to_device(K_all), synth.to_device(V_all))
            else:
                d_in = 128
                h = synth.normal_bf16((m * T, d_in), 1.0, seed, 51, step, 0)
                wk = synth.normal_bf16((H * D, d_in), (1.0 / d_in) ** 0.5, seed, 51, step, 1)
                wv = synth.normal_bf16((H * D, d_in), (1.0 / d_in) ** 0.5, seed, 51, step, 2)
                hd, wkd, wvd = synth.to_device(h), synth.to_device(wk), synth.to_device(wv)
                Kp, Vp = ll.kv_project(hd, wkd, wvd)
                cache.recache_from_hidden(0, hd, wkd, wvd)
                K_all, V_all = synth.to_bits(Kp).reshape(m * T, H, D), synth.to_bits(Vp).reshape(m * T, H, D)
            hist.recache(K_all, V_all)
            check_slots(cache, 0, hist, kv=kv)
        q, kc, vc = (synth.normal_bf16(shape, 1.0, seed, t, step) for t in range(3))
        out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
        rows = None if T < 1000 else sample_rows(n * T, T, seed=step)
        ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, kv=kv, shot=hist.shot, rows=rows)
        got = out if rows is None else synth.to_bits(out)[rows]
        compare_attention(got, ref, f"step {step} f0 {hist.f0} shot {hist.shot}")
        cache.append(0, synth.to_device(kc), synth.to_device(vc))
        hist.append(kc, vc)
        check_slots(cache, 0, hist, kv=kv)
        step += 1


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "mxfp4", "mxfp8"])
@pytest.mark.parametrize("S,Ss,W,T,D", [(3, 3, 6, 16, 64), (1, 4, 5, 33, 128), (0, 2, 3, 24, 64)])
def test_shot_rollout_with_recache(torch_gpu, kv, S, Ss, W, T, D):
    _log(f"shots kv={kv} S={S} Ss={Ss} W={W} T={T} D={D}")
    _rollout(torch_gpu, S, Ss, W, T, 2, D, kv, seed=700 + S * 10 + Ss,
             recache_at=(5, 9), fused_recache_at=(7, 12))


def test_shot_rollout_full_shape(torch_gpu):
    """12 heads x 128, 1560 tokens per frame: three cache runs at full size (the
    one-workgroup-per-CU split walk), sampled rows."""
    _rollout(torch_gpu, 3, 3, 12, 1560, 12, 128, "bf16", seed=777, fused_recache_at=(10,))
