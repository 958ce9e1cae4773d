"""GPU parity at the 1.3B-DiT shape: steady-state step, recache projection, int8 cache.

Steady step: 12 heads, head_dim 128, 1560 tokens per frame, chunk 3, sink 3, window
12, cache already full (10 seeded chunks appended, so the ring has wrapped), then 4
denoise passes with fresh N(0, 0.5^2) bf16 inputs (seed 1) and one append.
"""

import time

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from oracle import attention, bf16, gemm
from synth import configs

from helpers import History, check_slots, compare_attention, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()
    return torch


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _prefill(cache, hist, cfg, layer, n_chunks, tag):
    shape = (cfg.nq, cfg.heads, cfg.head_dim)
    for k in range(n_chunks):
        kb = synth.normal_bf16(shape, cfg.sigma, cfg.seed, tag, 1, layer, k)
        vb = synth.normal_bf16(shape, cfg.sigma, cfg.seed, tag, 2, layer, k)
        cache.append(layer, synth.to_device(kb), synth.to_device(vb))
        hist.append(kb, vb)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "mxfp4", "mxfp8"])
def test_steady_state_step(torch_gpu, kv):
    cfg = configs.STEADY
    if kv != "bf16":   # the low-bit workload's window
        cfg = configs.Workload(**{**cfg.__dict__, "window": configs.LONG_INT8.window, "kv_int8": True,
                                  "prefill_chunks": 9, "seed": configs.LONG_INT8.seed})
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    hist = History(S, W, T)
    _prefill(cache, hist, cfg, 0, cfg.prefill_chunks, 100)
    check_slots(cache, 0, hist, kv=kv)
    f0 = hist.f0
    shape = (cfg.nq, H, D)
    rows = sample_rows(cfg.nq, T, seed=cfg.seed)
    for p in range(cfg.passes):
        q, kc, vc = (synth.normal_bf16(shape, cfg.sigma, cfg.seed, t, 0, 0, p) for t in range(3))
        out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
        t0 = time.time()
        if p == 0:
            ref = attention.chunk_attention(q, kc, vc, hist, f0, S, W, T, kv=kv)
            mx, mn = compare_attention(out, ref, f"pass {p} (all rows)", scale_gate=True)
        else:
            ref = attention.chunk_attention(q, kc, vc, hist, f0, S, W, T, kv=kv, rows=rows)
            mx, mn = compare_attention(synth.to_bits(out)[rows], ref, f"pass {p} (sampled rows)", scale_gate=True)
        _log(f"steady kv={kv} pass {p}: max-abs {mx:.2e} mean-abs {mn:.2e} oracle {time.time() - t0:.1f}s")
    cache.append(0, synth.to_device(kc), synth.to_device(vc))
    hist.append(kc, vc)
    check_slots(cache, 0, hist, kv=kv)


def test_projection_identity_and_small_integers_bit_exact(torch_gpu):
    torch = torch_gpu
    n, d = 777, 256
    h = synth.normal_bf16((n, d), 1.0, 3, 500)
    eye = bf16.round_f32(np.eye(d, dtype=np.float32))
    K, V = ll.kv_project(synth.to_device(h), synth.to_device(eye), synth.to_device(eye))
    assert np.array_equal(synth.to_bits(K), h) and np.array_equal(synth.to_bits(V), h)
    # small integers: every fp32 partial sum is exact, so the bf16 outputs are unique.
    # 128, 384 and 768 outputs take the three tile shapes (256 x 128, 192 x 384 once
    # and twice); 777 tokens leave a ragged token tile in each.
    rng = np.random.default_rng(4)
    hi = bf16.round_f32(rng.integers(-8, 9, size=(n, 192)).astype(np.float32))
    for d_out in (128, 384, 768):
        wi = bf16.round_f32(rng.integers(-8, 9, size=(d_out, 192)).astype(np.float32))
        K, V = ll.kv_project(synth.to_device(hi), synth.to_device(wi), synth.to_device(wi))
        want = gemm.project_bf16(hi, wi)
        assert np.array_equal(synth.to_bits(K), want), d_out
        assert np.array_equal(synth.to_bits(V), want), d_out


def _projection_bound_violations(got_bits, h_bits, w_bits):
    """Count outputs outside the error bound of fp32 accumulation + one bf16 rounding.

    Any order of n fp32 additions of exact bf16 x bf16 products satisfies
    |s - exact| <= gamma_n * sum |h_k w_k|, gamma_n = n u / (1 - n u), u = 2^-24;
    rounding s to bf16 adds at most half an ulp of the result.  The oracle's own
    fp32 result obeys the same bound, so it is checked the same way.
    """
    h = bf16.to_f64(h_bits)
    w = bf16.to_f64(w_bits)
    exact = h @ w.T
    absum = np.abs(h) @ np.abs(w).T
    n = h.shape[1]
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    got = bf16.to_f64(got_bits)
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(got), 2.0 ** -126))) - 8)
    bound = half_ulp + gamma * absum
    bad = np.abs(got - exact) > bound
    return int(bad.sum()), float(np.abs(got - exact).max())


def _half_ulp_bf16(bits):
    """Half a bf16 ulp of each value."""
    x = np.abs(bf16.to_f64(bits))
    return np.exp2(np.floor(np.log2(np.maximum(x, 2.0 ** -126))) - 8)


def test_recache_all_30_layers_full_size(torch_gpu):
    """The recache workload at its stated size (LongLive explainer, dpshk.com, §三: the
    retained latents' K/V are recomputed under the new prompt and replace the old cache):
    30 layers, each holding 15 frames of NaN (a quiet-NaN bf16 prefill of 6 chunks, so
    any slot the recache misses stays NaN), each with its own hidden states h [23400][1536]
    ~ N(0, 1) and weights W_K, W_V [1536][1536] ~ N(0, 1/1536) (seed 3).  Per layer:
    K = h W_K^T, V = h W_V^T on the GPU against the oracle's fp32 GEMM: under 1% of the
    outputs may differ, and each difference must fit two fp32 summation orders of the same
    products (both within gamma_n sum |h_k w_k| of the exact sum, plus each one's bf16
    rounding); on layers 0, 15 and 29 every output is also checked against the exact fp64
    sum.  Then the rewrite of all 15 slots (bytes equal to the blocks passed, no
    NaN left), then the next chunk's attention on every layer (sampled rows of layers 0,
    15 and 29 against the oracle)."""
    torch = torch_gpu
    cfg = configs.RECACHE
    C, T, H, D, S, W, L = (cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window,
                           cfg.layers)
    hid = cfg.hidden
    cache = ll.Cache(L, H, D, T, S, W)
    nan = torch.full((C * T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    checked = {0, 15, L - 1}
    hists = {l: History(S, W, T) for l in checked}
    nan_bits = synth.to_bits(nan)
    for l in range(L):
        for k in range(cfg.prefill_chunks):
            cache.append(l, nan, nan)
            if l in hists:
                hists[l].append(nan_bits, nan_bits)
    n = min(cfg.prefill_chunks * C, S + W)
    assert n == S + W
    t0 = time.time()
    flips = 0
    for l in range(L):
        h = synth.normal_bf16_device((n * T, hid), 1.0, cfg.seed, 10, l)
        wk = synth.normal_bf16_device((hid, hid), (1.0 / hid) ** 0.5, cfg.seed, 11, l)
        wv = synth.normal_bf16_device((hid, hid), (1.0 / hid) ** 0.5, cfg.seed, 12, l)
        K, V = ll.kv_project(h, wk, wv)
        cache.recache(l, K.view(n * T, H, D), V.view(n * T, H, D))
        hb, kb, vb = synth.to_bits(h), synth.to_bits(K), synth.to_bits(V)
        habs = np.abs(bf16.to_f32(hb))
        gamma = hid * 2.0 ** -24 / (1 - hid * 2.0 ** -24)
        for got, w in ((kb, synth.to_bits(wk)), (vb, synth.to_bits(wv))):
            ref = gemm.project_bf16(hb, w)
            diff = got != ref
            flips += int(diff.sum())
            assert diff.mean() < 0.01, f"layer {l}: {diff.mean():.4f} of outputs differ from the oracle"
            if diff.any():   # another fp32 summation order of the same exact products
                absum = (habs @ np.abs(bf16.to_f32(w)).T)[diff].astype(np.float64) * (1 + 2.0 ** -20)
                d = np.abs(bf16.to_f64(got[diff]) - bf16.to_f64(ref[diff]))
                bound = 2 * gamma * absum + _half_ulp_bf16(got[diff]) + _half_ulp_bf16(ref[diff])
                assert (d <= bound).all(), f"layer {l}: {int((d > bound).sum())} differences beyond the bound"
            if l in checked:
                nbad, mx = _projection_bound_violations(got, hb, w)
                assert nbad == 0, f"layer {l}: {nbad} outputs outside the accumulation bound ({mx})"
        # every slot now holds its recache block: bytes equal to what was passed, no NaN left
        got = cache.slot_bytes(l)
        kk, vv = kb.reshape(n, T, H, D), vb.reshape(n, T, H, D)
        sf = cache.slot_frames(l)
        retained = sorted(f for f in sf if f >= 0)
        assert len(retained) == n
        for s_, f in enumerate(sf):
            idx = retained.index(f)
            assert np.array_equal(got["K"][s_].view(np.uint16), kk[idx]), (l, s_)
            assert np.array_equal(got["V"][s_].view(np.uint16), vv[idx]), (l, s_)
        assert not np.isnan(bf16.to_f32(got["K"].view(np.uint16))).any()
        if l in hists:
            hists[l].recache(kb.reshape(n * T, H, D), vb.reshape(n * T, H, D))
            assert sf == hists[l].model.slot_frame
    _log(f"recache of {L} layers checked in {time.time() - t0:.1f}s; {flips} outputs differ from the oracle's fp32 sums")
    shape = (cfg.nq, H, D)
    rows = sample_rows(cfg.nq, T, seed=3)
    for l in range(L):
        q, kc, vc = (synth.normal_bf16(shape, 0.5, cfg.seed, t, 20, l) for t in range(3))
        out = cache.attn(l, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
        if l in hists:
            ref = attention.chunk_attention(q, kc, vc, hists[l], hists[l].f0, S, W, T, rows=rows)
            mx, _ = compare_attention(synth.to_bits(out)[rows], ref, f"layer {l} after recache", scale_gate=True)
            _log(f"layer {l}: attention after recache max-abs {mx:.2e}")
    cache.close()


def test_frame_id_probe_at_full_shape(torch_gpu):
    """Frame-id probe at the 1.3B shape (12 heads x 128, 1560 tokens per frame, wrapped
    ring): K = 0 and V one-hot at d = frame id make every probability 1, so the output
    must be exactly (#visible tokens of frame d) / (#visible tokens)."""
    torch = torch_gpu
    from oracle import visibility
    T, H, D, S, W, C = 1560, 12, 128, 3, 12, 3
    cache = ll.Cache(1, H, D, T, S, W)
    f0 = 0
    for k in range(12):
        kz = torch.zeros((C * T, H, D), device="cuda", dtype=torch.bfloat16)
        v = torch.zeros((C * T, H, D), device="cuda", dtype=torch.bfloat16)
        for i in range(C):
            v[i * T:(i + 1) * T, :, (f0 + i) % D] = 1.0
        if k >= 5:
            q = synth.normal_bf16_device((C * T, H, D), 0.5, 77, k)
            out = cache.attn(0, q, kz, v)
            vis = visibility.visible_frames(f0, C, S, W)
            expect = np.zeros(D)
            for f in vis:
                expect[f % D] += T
            expect /= len(vis) * T
            got = bf16.to_f32(synth.to_bits(out)).astype(np.float64)
            want = bf16.to_f32(bf16.round_f32(expect.astype(np.float32))).astype(np.float64)
            assert np.abs(got - want[None, None, :]).max() <= np.abs(want).max() * 2 ** -7, (k, f0)
        cache.append(0, kz, v)
        f0 += C


@pytest.mark.parametrize("H,C,D,kv", [
    (8, 3, 128, "bf16"),    # 152 blocks: per-XCD split, 19 blocks per XCD
    (8, 4, 128, "bf16"),    # 200 blocks
    (12, 2, 128, "int8"),   # 156 blocks, quantised cache tiles in the split walk
    (16, 2, 128, "bf16"),   # 208 blocks
    (24, 1, 128, "fp8"),    # 168 blocks, one-frame chunk
    (12, 3, 64, "bf16"),    # 228 blocks of the head_dim-64 kernel (two query blocks per wave)
    (12, 4, 128, "bf16"),   # 300 blocks: more blocks than CUs, one workgroup per block
])
def test_attention_split_walk_shapes(torch_gpu, H, C, D, kv):
    """Block counts below the CU count take the per-XCD split walk (heads walk the first
    J - t key tiles, spare workgroups the tails, partials merged); sampled rows of every
    query tile against the oracle, including the first and last rows of each tile."""
    T, S, W = 1560, 3, 12
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    hist = History(S, W, T)
    kb = synth.normal_bf16((16 * T, H, D), 0.5, 900, H, C, D, 0)
    vb = synth.normal_bf16((16 * T, H, D), 0.5, 900, H, C, D, 1)
    cache.append(0, synth.to_device(kb), synth.to_device(vb))
    hist.append(kb, vb)
    nq = C * T
    q, kc, vc = (synth.normal_bf16((nq, H, D), 0.5, 901, H, C, D, t) for t in range(3))
    out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
    tile_rows = 256
    rows = set(sample_rows(nq, T, seed=H * 10 + C, n_random=24))
    for t0 in range(0, nq, tile_rows):
        rows |= {t0, min(t0 + tile_rows, nq) - 1}
    rows = sorted(rows)
    ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, kv=kv, rows=rows)
    mx, mn = compare_attention(synth.to_bits(out)[rows], ref, f"H={H} C={C} D={D} kv={kv}", scale_gate=True)
    _log(f"split walk H={H} C={C} D={D} kv={kv}: {len(rows)} rows, max-abs {mx:.2e} mean-abs {mn:.2e}")
    # the same chunk again: the arrival counters were reset by the merges
    out2 = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
    assert np.array_equal(synth.to_bits(out2), synth.to_bits(out))
