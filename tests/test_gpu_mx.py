"""GPU checks particular to the MX caches (MXFP4: E2M1 codes, MXFP8: E4M3 codes, each
with one power-of-two scale per block of 32 values): the quantising write on rows built
to hit every case of the rule, bit for bit against the oracle; attention bit-identical
to a bf16 cache's on exactly quantisable rows.  The MX caches also run through the
shared parity tests (toy rollout, recache, window recache, fused recache, maximum slot
count, steady step, peaked and tail-heavy full shapes, softmax paths, shot sinks, the
debug library)."""

import time

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from oracle import attention, bf16, quant

from helpers import History, check_slots

pytestmark = pytest.mark.gpu

MIDPOINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
_E4M3 = quant.e4m3_values()
E4M3_MIDPOINTS = list((_E4M3[:-1] + _E4M3[1:]) / 2)   # 126 midpoints, all bf16 values


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()
    return torch


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _edge_block(kind, rng, k, huge, kv, j):
    """32 float32 values of one block (the j-th of its kind), scaled by 2^k where it
    applies (rounded to bf16 by the caller)."""
    b = rng.standard_normal(32).astype(np.float32)
    if kind == 0:                      # all zero, with signed zeros
        b = np.where(np.arange(32) % 3 == 0, -0.0, 0.0).astype(np.float32)
    elif kind == 1 and kv == "mxfp4":  # every midpoint, both signs, block max 6 * 2^k
        vals = [6.0] + MIDPOINTS + [-m for m in MIDPOINTS] + [4.0, -3.0, 0.5, -0.5, 0.0, -0.0, 1.0, -1.5]
        vals += [0.125, -0.125] * 5                         # below the smallest code: +-0
        b = np.array(vals[:32], dtype=np.float32) * np.float32(2.0 ** k)
    elif kind == 1:                    # 31 of the E4M3 midpoints (a different run per block), max 448 * 2^k
        mids = [E4M3_MIDPOINTS[(31 * j + t) % len(E4M3_MIDPOINTS)] * (-1) ** t for t in range(31)]
        b = np.array([448.0] + mids, dtype=np.float32) * np.float32(2.0 ** k)
    elif kind == 2 and kv == "mxfp4":  # block max 7.5 * 2^k: 6.5 and 7 saturate to 6
        b = np.array([7.5, 6.5, -7.0, 6.0, -6.25] + [0.3] * 27, dtype=np.float32) * np.float32(2.0 ** k)
    elif kind == 2:                    # block max 480 * 2^k: 460 and -500 saturate to 448
        b = np.array([480.0, 460.0, -500.0, 448.0, -456.0] + [3.0] * 27, dtype=np.float32) * np.float32(2.0 ** k)
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


def _edge_rows(T, H, D, seed, huge, kv="mxfp4", k_hi=30):
    """Rows of edge blocks; block exponents k drawn from [-30, k_hi)."""
    rng = np.random.default_rng(seed)
    x = np.empty((T, H, D), dtype=np.float32)
    j = 0
    for t in range(T):
        for h in range(H):
            for blk in range(D // 32):
                kind = (t + 3 * h + 5 * blk) % 8
                x[t, h, 32 * blk:32 * (blk + 1)] = _edge_block(kind, rng, int(rng.integers(-30, k_hi)), huge, kv, j)
                j += 1
    return x


@pytest.mark.parametrize("kv", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("huge", [125, 10])
def test_mx_quantisation_edge_rows_bit_exact(torch_gpu, D, huge, kv):
    """Blocks that are all zero (signed zeros), hold the element format's midpoints (ties
    to the even code: all 7 E2M1 ones, or runs of the 126 E4M3 ones), saturate (block max
    7.5 * 2^k, or 480 * 2^k), are tiny (bf16 subnormals: the exponent's lower bound),
    huge (2^125: the top of the bf16 range), hold one value, or have a power-of-two max,
    beside Gaussian blocks: codes and block scales bit-exact against the oracle after
    every append.  With huge = 10 (and block exponents below 0) the attention over these
    slots is compared with the oracle too; with 2^125 it is not: keys that large put the scores
    far outside the kernel's input domain (scores q.k/sqrt(D) below 2^14, where the
    fused exponent argument fma(s, log2(e)/sqrt(D), -max) is exact to well under the
    bf16 rounding of the probabilities; near 2^24 and above, the rounding of s times the
    factor is itself an ulp of several units and the weights lose all meaning)."""
    T, H, S, W = 24, 2, 2, 3
    # the codes-only variant scales blocks up to 2^29; the one whose attention is checked
    # keeps them below 2^0 (E4M3 blocks reach 500 * 2^k), inside the attention's domain
    x = _edge_rows(T, H, D, 31 + D, huge, kv, k_hi=30 if huge > 100 else 0)
    frames = synth.f32_to_bf16_bits(x)
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    hist = History(S, W, T)
    for k in range(4):
        kb = frames if k % 2 == 0 else synth.f32_to_bf16_bits(-x)
        vb = synth.f32_to_bf16_bits(x[::-1].copy())
        cache.append(0, synth.to_device(kb), synth.to_device(vb))
        hist.append(kb, vb)
        check_slots(cache, 0, hist, kv=kv)
    if huge > 100:
        _log(f"{kv} edge rows D={D} huge=2^{huge}: codes and scales bit-exact")
        return
    q = synth.normal_bf16((T, H, D), 1.0, 32, D, 0)
    kc = synth.normal_bf16((T, H, D), 1.0, 32, D, 1)
    vc = synth.normal_bf16((T, H, D), 1.0, 32, D, 2)
    out = cache.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc))
    ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, kv=kv)
    got = bf16.to_f32(synth.to_bits(out)).astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref.astype(np.float64))
    assert err.max() <= 2.0 ** -7 * np.abs(ref).max(), (err.max(), np.abs(ref).max())
    _log(f"{kv} edge rows D={D} huge=2^{huge}: codes and scales bit-exact; attention max err {err.max():.3g}")


@pytest.mark.parametrize("kv", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("D", [64, 128])
def test_mx_attention_bit_identical_to_bf16_on_exact_rows(torch_gpu, D, kv):
    """History rows whose MX quantisation is exact (element-format values times 2^k per
    block, each block holding a value that fixes the exponent at k: +-4 or +-6 for E2M1,
    256..448 for E4M3): the widened tiles are then the bf16 tiles, so the MX cache's
    attention output must equal a bf16 cache's bit for bit on the same inputs (the
    widening, scales and tile order are all exercised)."""
    T, H, S, W, C = 32, 2, 2, 4, 2
    rng = np.random.default_rng(40 + D)
    if kv == "mxfp4":
        grid, tops = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]), np.array([4.0, 6.0])
    else:
        grid, tops = _E4M3, _E4M3[120:]

    def exact_rows(n):
        k = rng.integers(-4, 3, size=(n, H, D // 32)) - (0 if kv == "mxfp4" else 8)
        mags = grid[rng.integers(0, len(grid), size=(n, H, D // 32, 32))]
        mags[..., 0] = tops[rng.integers(0, len(tops), size=(n, H, D // 32))]
        x = mags * rng.choice([-1.0, 1.0], size=mags.shape) * np.ldexp(1.0, k)[..., None]
        return synth.f32_to_bf16_bits(x.reshape(n, H, D).astype(np.float32))

    caches = {name: ll.Cache(1, H, D, T, S, W, kv_dtype=name) for name in ("bf16", kv)}
    hist = History(S, W, T)
    for chunk in range(6):
        q = synth.normal_bf16((C * T, H, D), 1.0, 41, D, chunk, 0)
        kc, vc = exact_rows(C * T), exact_rows(C * T)
        outs = {name: synth.to_bits(c.attn(0, synth.to_device(q), synth.to_device(kc), synth.to_device(vc)))
                for name, c in caches.items()}
        same = outs["bf16"] == outs[kv]
        assert same.all(), (f"D={D} chunk {chunk}: {int((~same).sum())} outputs differ, "
                            f"e.g. {np.argwhere(~same)[:4].tolist()}")
        for c in caches.values():
            c.append(0, synth.to_device(kc), synth.to_device(vc))
        hist.append(kc, vc)
        check_slots(caches[kv], 0, hist, kv=kv)
    _log(f"{kv} exact rows D={D}: bit-identical to the bf16 cache over 6 chunks")
