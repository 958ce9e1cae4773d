"""GPU checks particular to the MXFP4 cache (E2M1 codes with one power-of-two scale per
block of 32 values): the quantising write on rows built to hit every case of the rule,
bit for bit against the oracle, and the fused projection's refusal of this format.
The MXFP4 cache also runs through the shared parity tests (toy rollout, recache,
window recache, maximum slot count, steady step, peaked and tail-heavy full shapes,
softmax paths, shot sinks)."""

import time

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from oracle import attention, bf16

from helpers import History, check_slots, compare_attention

pytestmark = pytest.mark.gpu

MIDPOINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()
    return torch


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _edge_block(kind, rng, k, huge):
    """32 float32 values of one block, scaled by 2^k where it applies (rounded to bf16
    by the caller)."""
    b = rng.standard_normal(32).astype(np.float32)
    if kind == 0:                      # all zero, with signed zeros
        b = np.where(np.arange(32) % 3 == 0, -0.0, 0.0).astype(np.float32)
    elif kind == 1:                    # every midpoint, both signs, block max 6 * 2^k
        vals = [6.0] + MIDPOINTS + [-m for m in MIDPOINTS] + [4.0, -3.0, 0.5, -0.5, 0.0, -0.0, 1.0, -1.5]
        vals += [0.125, -0.125] * 5                         # below the smallest code: +-0
        b = np.array(vals[:32], dtype=np.float32) * np.float32(2.0 ** k)
    elif kind == 2:                    # block max 7.5 * 2^k: 6.5 and 7 saturate to 6
        b = np.array([7.5, 6.5, -7.0, 6.0, -6.25] + [0.3] * 27, dtype=np.float32) * np.float32(2.0 ** k)
    elif kind == 3:                    # tiny: bf16 subnormals and values near 2^-126
        b = b * np.float32(2.0 ** -129)
    elif kind == 4:                    # huge (with 2^125 the block exponent reaches its top, 125)
        b = b * np.float32(2.0 ** huge)
        b[0] = np.float32(1.5 * 2.0 ** (huge + 2))
    elif kind == 5:                    # one non-zero value
        b = np.zeros(32, dtype=np.float32)
        b[k % 32] = -3.0
    elif kind == 6:                    # block max a power of two (the exponent's edge)
        b = np.clip(b, -1.0, 1.0)
        b[0] = 4.0
    return b


def _edge_rows(T, H, D, seed, huge):
    rng = np.random.default_rng(seed)
    x = np.empty((T, H, D), dtype=np.float32)
    for t in range(T):
        for h in range(H):
            for blk in range(D // 32):
                kind = (t + 3 * h + 5 * blk) % 8
                x[t, h, 32 * blk:32 * (blk + 1)] = _edge_block(kind, rng, int(rng.integers(-30, 30)), huge)
    return x


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("huge", [125, 10])
def test_mxfp4_quantisation_edge_rows_bit_exact(torch_gpu, D, huge):
    """Blocks that are all zero (signed zeros), hold every E2M1 midpoint (ties to the
    even code), saturate (block max 7.5 * 2^k), are tiny (bf16 subnormals: the exponent's
    lower bound), huge (2^125: the top of the bf16 range), hold one value, or have a
    power-of-two max, beside Gaussian blocks: codes and block scales bit-exact against
    the oracle after every append.  With huge = 10 the attention over these slots is
    compared with the oracle too; with 2^125 it is not: keys that large put the scores
    far outside the kernel's input domain (|scores| in log2 units below 2^15, where the
    fused exponent argument fma(s, log2(e)/sqrt(D), -max) is exact to well under the
    bf16 rounding of the probabilities; near 2^24 and above, the rounding of s times the
    factor is itself an ulp of several units and the weights lose all meaning)."""
    T, H, S, W = 24, 2, 2, 3
    x = _edge_rows(T, H, D, 31 + D, huge)
    frames = synth.f32_to_bf16_bits(x)
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype="mxfp4")
    hist = History(S, W, T)
    for k in range(4):
        kb = frames if k % 2 == 0 else synth.f32_to_bf16_bits(-x)
        vb = synth.f32_to_bf16_bits(x[::-1].copy())
        cache.append(0, synth.to_device(kb), synth.to_device(vb))
        hist.append(kb, vb)
        check_slots(cache, 0, hist, kv="mxfp4")
    if huge > 100:
        _log(f"mxfp4 edge rows D={D} huge=2^{huge}: codes and scales bit-exact")
        return
    q = synth.normal_bf16((T, H, D), 1.0, 32, D, 0)
    kc = synth.normal_bf16((T, H, D), 1.0, 32, D, 1)
    vc = synth.normal_bf16((T, H, D), 1.0, 32, D, 2)
    out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
    ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, kv="mxfp4")
    got = bf16.to_f32(synth.to_bits(out)).astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref.astype(np.float64))
    assert err.max() <= 2.0 ** -7 * np.abs(ref).max(), (err.max(), np.abs(ref).max())
    _log(f"mxfp4 edge rows D={D} huge=2^{huge}: codes and scales bit-exact; attention max err {err.max():.3g}")


def test_mxfp4_fused_recache_is_refused(torch_gpu):
    T, H, D, S, W, C = 16, 2, 64, 3, 6, 3
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype="mxfp4")
    kb = synth.normal_bf16((C * T, H, D), 1.0, 33, 0)
    cache.append(0, synth.to_device(kb), synth.to_device(kb))
    d_in = 128
    h = synth.to_device(synth.normal_bf16((C * T, d_in), 1.0, 33, 1))
    w = synth.to_device(synth.normal_bf16((H * D, d_in), 0.1, 33, 2))
    with pytest.raises(ll.LLError) as e:
        cache.recache_from_hidden(0, h, w, w)
    assert e.value.status == ll.LL_ERR_INVALID
    # the cache is untouched and still usable
    hist = History(S, W, T)
    hist.append(kb, kb)
    check_slots(cache, 0, hist, kv="mxfp4")
    q = synth.normal_bf16((C * T, H, D), 1.0, 33, 3)
    out = cache.attn(0, synth.to_device(q), synth.to_device(kb), synth.to_device(kb))
    ref = attention.chunk_attention(q, kb, kb, hist, hist.f0, S, W, T, kv="mxfp4")
    compare_attention(out, ref, "mxfp4 after a refused fused recache")


@pytest.mark.parametrize("D", [64, 128])
def test_mxfp4_attention_bit_identical_to_bf16_on_exact_rows(torch_gpu, D):
    """History rows whose MXFP4 quantisation is exact (grid values times 2^k per block,
    each block holding a +-4 or +-6 times 2^k): the widened tiles are then the bf16
    tiles, so the MXFP4 cache's attention output must equal a bf16 cache's bit for bit
    on the same inputs (the widening, scales and tile order are all exercised)."""
    T, H, S, W, C = 32, 2, 2, 4, 2
    rng = np.random.default_rng(40 + D)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

    def exact_rows(n):
        k = rng.integers(-4, 3, size=(n, H, D // 32))
        mags = grid[rng.integers(0, 8, size=(n, H, D // 32, 32))]
        mags[..., 0] = np.array([4.0, 6.0])[rng.integers(0, 2, size=(n, H, D // 32))]
        x = mags * rng.choice([-1.0, 1.0], size=mags.shape) * np.ldexp(1.0, k)[..., None]
        return synth.f32_to_bf16_bits(x.reshape(n, H, D).astype(np.float32))

    caches = {kv: ll.Cache(1, H, D, T, S, W, kv_dtype=kv) for kv in ("bf16", "mxfp4")}
    hist = History(S, W, T)
    for chunk in range(6):
        q = synth.normal_bf16((C * T, H, D), 1.0, 41, D, chunk, 0)
        kc, vc = exact_rows(C * T), exact_rows(C * T)
        outs = {kv: synth.to_bits(c.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc)))
                for kv, c in caches.items()}
        same = outs["bf16"] == outs["mxfp4"]
        assert same.all(), (f"D={D} chunk {chunk}: {int((~same).sum())} outputs differ, "
                            f"e.g. {np.argwhere(~same)[:4].tolist()}")
        for c in caches.values():
            c.append(0, synth.to_device(kc), synth.to_device(vc))
        hist.append(kc, vc)
        check_slots(caches["mxfp4"], 0, hist, kv="mxfp4")
    _log(f"mxfp4 exact rows D={D}: bit-identical to the bf16 cache over 6 chunks")
