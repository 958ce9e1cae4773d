"""GPU parity on the tiny streaming toy and on the cache's edge cases.

Toy workload: 1 layer, 2 heads, head_dim 64, 16 tokens per frame, chunk 3, sink 3,
window 6; 12 chunks with 2 denoise passes each, then an append.  Inputs are fp32
N(0, 1) from seed 0 rounded to bf16.  Every attention output is compared with the
oracle in full, and after every append the slot contents are compared bit for bit.
"""

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from oracle import attention, bf16, quant, visibility
from synth import configs

from helpers import History, check_slots, compare_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()   # the HIP library must be there; no fallback
    return torch


def _chunk_inputs(cfg, k, p, sigma=None):
    shape = (cfg.nq, cfg.heads, cfg.head_dim)
    s = cfg.sigma if sigma is None else sigma
    return tuple(synth.normal_bf16(shape, s, cfg.seed, t, 0, k, p) for t in range(3))


def _rollout(torch, cfg, kv="bf16", chunk_sizes=None, check_every_pass=True):
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    hist = History(S, W, T)
    for k in range(cfg.chunks):
        f0 = hist.f0
        for p in range(cfg.passes):
            q, kc, vc = _chunk_inputs(cfg, k, p)
            out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
            if check_every_pass or p == cfg.passes - 1:
                ref = attention.chunk_attention(q, kc, vc, hist, f0, S, W, T, kv=kv)
                compare_attention(out, ref, f"chunk {k} pass {p}")
        cache.append(0, synth.to_device(kc), synth.to_device(vc))
        hist.append(kc, vc)
        check_slots(cache, 0, hist, kv=kv)
    return cache, hist


def test_toy_rollout_bf16(torch_gpu):
    _rollout(torch_gpu, configs.TOY)


def test_toy_rollout_int8(torch_gpu):
    _rollout(torch_gpu, configs.TOY, kv="int8")


def test_toy_rollout_fp8(torch_gpu):
    _rollout(torch_gpu, configs.TOY, kv="fp8")


def test_toy_rollout_mxfp4(torch_gpu):
    _rollout(torch_gpu, configs.TOY, kv="mxfp4")


def test_toy_rollout_mxfp8(torch_gpu):
    _rollout(torch_gpu, configs.TOY, kv="mxfp8")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S,W,n_list", [
    (3, 6, [3] * 12),
    (0, 4, [3] * 8),              # no sink: plain sliding window
    (2, 0, [1, 1, 1, 3]),         # sink only
    (3, 6, [20, 3, 1, 9]),        # appends longer than the window
    (1, 2, [1] * 10),
])
def test_frame_id_probe(torch_gpu, D, S, W, n_list):
    """K = 0 and V one-hot at d = frame id: every score is 0, every probability 1,
    so out[d] = (#visible tokens of frame d) / (#visible tokens) exposes exactly
    which frames the kernel read."""
    torch = torch_gpu
    T, H = 40, 3
    cache = ll.Cache(1, H, D, T, S, W)
    f0 = 0
    for n in n_list:
        frames = np.arange(f0, f0 + n)
        q = torch.randn((n * T, H, D), device="cuda").to(torch.bfloat16)
        kz = torch.zeros((n * T, H, D), device="cuda", dtype=torch.bfloat16)
        v = torch.zeros((n * T, H, D), device="cuda", dtype=torch.bfloat16)
        for i, f in enumerate(frames):
            v[i * T:(i + 1) * T, :, f % D] = 1.0
        out = cache.attn(0, q, kz, v)
        vis = visibility.visible_frames(f0, n, S, W)
        expect = np.zeros(D)
        for f in vis:
            expect[f % D] += T
        expect /= len(vis) * T
        got = bf16.to_f32(synth.to_bits(out)).astype(np.float64)
        want = bf16.to_f32(bf16.round_f32(expect.astype(np.float32))).astype(np.float64)
        assert np.abs(got - want[None, None, :]).max() <= np.abs(want).max() * 2 ** -7, (f0, n)
        cache.append(0, kz, v)
        f0 += n


def test_append_longer_than_window_and_sink_only(torch_gpu):
    torch = torch_gpu
    T, H, D = 24, 2, 64
    for S, W, ns in [(3, 6, [20, 1, 13]), (2, 0, [1, 4, 2]), (0, 5, [12, 2, 7]), (4, 3, [2, 1, 9])]:
        cache = ll.Cache(1, H, D, T, S, W)
        hist = History(S, W, T)
        for j, n in enumerate(ns):
            kb = synth.normal_bf16((n * T, H, D), 1.0, 77, S, W, j, 0)
            vb = synth.normal_bf16((n * T, H, D), 1.0, 77, S, W, j, 1)
            cache.append(0, synth.to_device(kb), synth.to_device(vb))
            hist.append(kb, vb)
            check_slots(cache, 0, hist)
            q = synth.normal_bf16((3 * T, H, D), 1.0, 78, S, W, j)
            kc = synth.normal_bf16((3 * T, H, D), 1.0, 79, S, W, j)
            vc = synth.normal_bf16((3 * T, H, D), 1.0, 80, S, W, j)
            out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
            ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T)
            compare_attention(out, ref, f"S={S} W={W} step {j}")


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "mxfp4", "mxfp8"])
def test_recache_overwrites_every_slot(torch_gpu, kv):
    """Prefill with NaN K/V, recache with finite tensors: no stale (NaN) slot may
    survive, the bytes must be exactly the recache blocks, and attention must match
    the oracle fed the recache tensors."""
    torch = torch_gpu
    T, H, D, S, W, C = 32, 2, 128, 3, 6, 3
    kv_int8 = kv != "bf16"
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    hist = History(S, W, T)
    nan = np.full((C * T, H, D), 0x7FC0, dtype=np.uint16)   # bf16 quiet NaN
    for k in range(5):
        if kv_int8:   # codes of NaN rows are undefined; poison through the chunk path
            kb = synth.normal_bf16((C * T, H, D), 1.0, 90, k, 0)
            cache.append(0, synth.to_device(kb), synth.to_device(kb))
            hist.append(kb, kb)
        else:
            cache.append(0, synth.to_device(nan), synth.to_device(nan))
            hist.append(nan, nan)
    n = min(hist.f0, S + W)
    K_all = synth.normal_bf16((n * T, H, D), 1.0, 91, 0)
    V_all = synth.normal_bf16((n * T, H, D), 1.0, 91, 1)
    cache.recache(0, synth.to_device(K_all), synth.to_device(V_all))
    hist.recache(K_all, V_all)
    check_slots(cache, 0, hist, kv=kv)
    got = cache.slot_bytes(0)
    if not kv_int8:
        assert not np.isnan(bf16.to_f32(got["K"].view(np.uint16))).any()
        assert not np.isnan(bf16.to_f32(got["V"].view(np.uint16))).any()
    q = synth.normal_bf16((C * T, H, D), 1.0, 92, 0)
    kc = synth.normal_bf16((C * T, H, D), 1.0, 92, 1)
    vc = synth.normal_bf16((C * T, H, D), 1.0, 92, 2)
    out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
    ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, kv=kv)
    compare_attention(out, ref, "after recache")
    # wrong frame count is a state error, not a launch
    with pytest.raises(ll.LLError) as e:
        cache.recache(0, synth.to_device(K_all[:T]), synth.to_device(V_all[:T]))
    assert e.value.status == ll.LL_ERR_STATE


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "mxfp4", "mxfp8"])
def test_recache_window_keeps_sink(torch_gpu, kv):
    """Window-only recache (techwalker.com article, §六): the window frames' slots get the
    new blocks (oracle.ring's window order), the sink keeps its bytes, and the next
    chunk's attention sees the new window and the old sink."""
    T, H, D, S, W, C = 16, 2, 64, 3, 6, 3
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    hist = History(S, W, T)
    for k in range(4):
        kb = synth.normal_bf16((C * T, H, D), 1.0, 93, k, 0)
        vb = synth.normal_bf16((C * T, H, D), 1.0, 93, k, 1)
        cache.append(0, synth.to_device(kb), synth.to_device(vb))
        hist.append(kb, vb)
    n = len(hist.model.window_frames())
    K_w = synth.normal_bf16((n * T, H, D), 1.0, 94, 0)
    V_w = synth.normal_bf16((n * T, H, D), 1.0, 94, 1)
    cache.recache_window(0, synth.to_device(K_w), synth.to_device(V_w))
    hist.recache_window(K_w, V_w)
    check_slots(cache, 0, hist, kv=kv)
    for p in range(2):
        q, kc, vc = (synth.normal_bf16((C * T, H, D), 1.0, 95, p, t) for t in range(3))
        out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
        ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, kv=kv)
        compare_attention(out, ref, f"after window recache, pass {p}")
    with pytest.raises(ll.LLError) as e:
        cache.recache_window(0, synth.to_device(K_w[:T]), synth.to_device(V_w[:T]))
    assert e.value.status == ll.LL_ERR_STATE


def test_empty_cache_first_chunk_and_ragged_lengths(torch_gpu):
    # first chunk (nothing cached) and query counts that are not tile multiples
    for T in (1, 7, 33, 130):
        cache = ll.Cache(1, 3, 128, T, 3, 6)
        hist = History(3, 6, T)
        for k in range(4):
            q = synth.normal_bf16((3 * T, 3, 128), 1.0, 95, T, k, 0)
            kc = synth.normal_bf16((3 * T, 3, 128), 1.0, 95, T, k, 1)
            vc = synth.normal_bf16((3 * T, 3, 128), 1.0, 95, T, k, 2)
            out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
            ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, 3, 6, T)
            compare_attention(out, ref, f"T={T} chunk {k}")
            cache.append(0, synth.to_device(kc), synth.to_device(vc))
            hist.append(kc, vc)


@pytest.mark.parametrize("kv", ["int8", "fp8"])
def test_quantisation_edge_rows_bit_exact(torch_gpu, kv):
    """Rows built to hit every branch of the int8 / fp8 rule: exact ties (.5 for int8;
    E4M3 midpoints, normal and subnormal, for fp8 with absmax 448 so that the quotient
    is the value itself), +-absmax, all-zero rows, a single non-zero element, tiny
    (~2^-110) and huge (~2^121, x*M overflows) magnitudes, and ordinary Gaussian rows;
    codes and scales must equal the oracle's."""
    T, H, D, S, W = 24, 2, 128, 2, 3
    rng = np.random.default_rng(21)
    x = rng.standard_normal((T, H, D)).astype(np.float32)
    ties = np.zeros(D, dtype=np.float32)
    if kv == "int8":
        ties[:8] = [254.0, 1.0, 3.0, 5.0, -1.0, -3.0, -5.0, -254.0]
        ties[8:] = (2 * rng.integers(-60, 60, D - 8) + 1).astype(np.float32)
    else:
        v = quant.e4m3_values()
        mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)          # 126 midpoints, bf16-exact
        ties[0] = 448.0
        ties[1:1 + len(mids)] = mids * np.where(np.arange(len(mids)) % 2, -1, 1).astype(np.float32)
        ties[127] = -448.0
    for t in range(T):
        kind = t % 8
        if kind == 1:
            x[t] = 0.0
        elif kind == 2:
            x[t] = ties
        elif kind == 3:
            x[t] *= np.float32(2.0 ** -110)
        elif kind == 4:
            x[t] *= np.float32(2.0 ** 121)
        elif kind == 5:
            x[t] = 0.0
            x[t, :, t % D] = -3.5
        elif kind == 6:
            x[t, 0] *= np.float32(2.0 ** -20)
            x[t, 1] *= np.float32(2.0 ** 20)
    frames = synth.f32_to_bf16_bits(x)
    assert (bf16.to_f32(synth.f32_to_bf16_bits(ties)) == ties).all()   # the tie row is bf16-exact
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    hist = History(S, W, T)
    for k in range(4):
        kb = frames if k % 2 == 0 else synth.f32_to_bf16_bits(-x)
        vb = synth.f32_to_bf16_bits(x[::-1].copy())
        cache.append(0, synth.to_device(kb), synth.to_device(vb))
        hist.append(kb, vb)
        check_slots(cache, 0, hist, kv=kv)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "mxfp4", "mxfp8"])
def test_maximum_slot_count(torch_gpu, kv):
    """S + W = 128 slots (the largest cache the library accepts): sink 8, window 120,
    16 tokens per frame, 2 heads x 128.  50 chunks of 3 frames wrap the 120-slot ring
    once (f0 = 150); the attention of the chunks that see the most keys (128 cached frames
    plus the own chunk: 2096 keys, 33 key tiles) is compared with the oracle in full, and
    the slot contents bit for bit at the end."""
    T, H, D, S, W, C = 16, 2, 128, 8, 120, 3
    assert S + W == ll.MAX_SLOTS
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    hist = History(S, W, T)
    shape = (C * T, H, D)
    for k in range(50):
        q, kc, vc = (synth.normal_bf16(shape, 1.0, 780, t, k) for t in range(3))
        if hist.f0 >= S + W or k in (0, 1, 2):
            out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
            ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, kv=kv)
            compare_attention(out, ref, f"max slots kv={kv} chunk {k} f0={hist.f0}")
        cache.append(0, synth.to_device(kc), synth.to_device(vc))
        hist.append(kc, vc)
    assert hist.f0 == 150
    check_slots(cache, 0, hist, kv=kv)
