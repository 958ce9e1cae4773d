"""Pins for oracle.attention (CPU only).

The oracle is compared with torch's scaled_dot_product_attention (a library
routine) in the two limits where sink+window attention reduces to a textbook
form, with a float64 triple loop, with closed forms, and with invariants.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import attention, bf16, visibility


def _rollout_inputs(chunks, C, T, H, D, seed, sigma=1.0):
    out = []
    for k in range(chunks):
        q = synth.normal_bf16((C * T, H, D), sigma, seed, 0, k)
        kk = synth.normal_bf16((C * T, H, D), sigma, seed, 1, k)
        v = synth.normal_bf16((C * T, H, D), sigma, seed, 2, k)
        out.append((q, kk, v))
    return out


def _history_from(chunks, C, T):
    def history(f):
        k, r = divmod(f, C)
        _, kk, v = chunks[k]
        return kk[r * T:(r + 1) * T], v[r * T:(r + 1) * T]
    return history


def _sdpa(q, k, v, mask):
    # q [nq][D], k/v [nk][D] float64; mask [nq][nk] bool (True = attend)
    return F.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], attn_mask=torch.from_numpy(mask)[None, None],
    )[0, 0].numpy()


@pytest.mark.parametrize("S", [0, 3])
def test_large_window_equals_full_block_causal(S):
    C, T, H, D, n = 3, 4, 2, 16, 6
    ch = _rollout_inputs(n, C, T, H, D, seed=11)
    Qall = np.concatenate([bf16.to_f64(c[0]) for c in ch])
    Kall = np.concatenate([bf16.to_f64(c[1]) for c in ch])
    Vall = np.concatenate([bf16.to_f64(c[2]) for c in ch])
    chunk_of = np.repeat(np.arange(n), C * T)
    block_causal = chunk_of[:, None] >= chunk_of[None, :]
    hist = _history_from(ch, C, T)
    for k in range(n):
        got = attention.chunk_attention(*ch[k], hist, k * C, S, 10_000, T, dtype=np.float64)
        rows = slice(k * C * T, (k + 1) * C * T)
        for h in range(H):
            ref = _sdpa(Qall[rows, h], Kall[:, h], Vall[:, h], block_causal[rows])
            np.testing.assert_allclose(got[:, h], ref, rtol=0, atol=1e-12)


def test_no_sink_equals_sliding_window_on_sliced_keys():
    C, T, H, D, n, W = 3, 4, 2, 16, 7, 5
    ch = _rollout_inputs(n, C, T, H, D, seed=12)
    Kall = np.concatenate([bf16.to_f64(c[1]) for c in ch])
    Vall = np.concatenate([bf16.to_f64(c[2]) for c in ch])
    hist = _history_from(ch, C, T)
    for k in range(n):
        f0 = k * C
        got = attention.chunk_attention(*ch[k], hist, f0, 0, W, T, dtype=np.float64)
        lo, hi = max(0, f0 - W) * T, (f0 + C) * T       # the last W frames plus the chunk
        q = bf16.to_f64(ch[k][0])
        full = np.ones((C * T, hi - lo), dtype=bool)
        for h in range(H):
            ref = _sdpa(q[:, h], Kall[lo:hi, h], Vall[lo:hi, h], full)
            np.testing.assert_allclose(got[:, h], ref, rtol=0, atol=1e-12)


def test_rows_sum_to_one_and_masked_weights_are_zero():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((7, 8)), rng.standard_normal((20, 8))
    mask = rng.random((7, 20)) < 0.6
    mask[:, 0] = True
    P = attention.attention_probabilities(q, k, mask, 0.3)
    assert np.abs(P.sum(axis=1) - 1).max() <= 1e-12
    assert (P[~mask] == 0).all() and (P >= 0).all()


def test_key_permutation_invariance():
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((9, 16)), rng.standard_normal((40, 16)), rng.standard_normal((40, 16))
    mask = rng.random(40) < 0.7
    perm = rng.permutation(40)
    a = attention.masked_attention(q, k, v, mask, 0.25, np.float64)
    b = attention.masked_attention(q, k[perm], v[perm], mask[perm], 0.25, np.float64)
    assert np.abs(a - b).max() <= 1e-12


def test_fp32_oracle_matches_fp64_bruteforce_on_toy_size():
    # toy workload sizes: 48 queries, up to (9 + 3) * 16 = 192 keys, D = 64
    rng = np.random.default_rng(7)
    q = bf16.to_f32(synth.normal_bf16((48, 64), 1.0, 99, 0))
    k = bf16.to_f32(synth.normal_bf16((192, 64), 1.0, 99, 1))
    v = bf16.to_f32(synth.normal_bf16((192, 64), 1.0, 99, 2))
    mask = rng.random(192) < 0.8
    scale = attention.softmax_scale(64)
    got = attention.masked_attention(q, k, v, mask, scale, np.float32)
    ref = attention.attention_bruteforce_f64(q[:12], k, v, mask, 1.0 / 8.0)
    assert np.abs(got[:12] - ref).max() <= 1e-5


def test_zero_keys_give_mean_of_visible_values_and_single_key_gives_its_value():
    rng = np.random.default_rng(8)
    v = rng.standard_normal((30, 8))
    mask = rng.random(30) < 0.5
    mask[3] = True
    out = attention.masked_attention(rng.standard_normal((4, 8)), np.zeros((30, 8)), v, mask, 0.5, np.float64)
    np.testing.assert_allclose(out, np.broadcast_to(v[mask].mean(axis=0), out.shape), atol=1e-14)
    one = np.zeros(30, dtype=bool)
    one[17] = True
    out = attention.masked_attention(rng.standard_normal((4, 8)), rng.standard_normal((30, 8)), v, one, 0.5, np.float64)
    np.testing.assert_allclose(out, np.broadcast_to(v[17], out.shape), atol=0)


@pytest.mark.parametrize("S,W", [(3, 6), (0, 4), (2, 0), (3, 12)])
def test_frame_id_probe_counts_visible_frames_per_residue(S, W):
    """K = 0 and V one-hot at d = frame mod D: out[d] = (#visible tokens with
    frame = d mod D) / (#visible tokens)."""
    C, T, H, D = 3, 5, 1, 16
    n = 9

    def onehot_frame(f):
        x = np.zeros((T, H, D), dtype=np.float32)
        x[:, :, f % D] = 1.0
        return bf16.round_f32(x)

    zeros = bf16.round_f32(np.zeros((T, H, D), dtype=np.float32))
    hist = lambda f: (zeros, onehot_frame(f))
    for k in range(n):
        f0 = k * C
        own_v = np.concatenate([onehot_frame(f0 + i) for i in range(C)])
        own_k = np.concatenate([zeros] * C)
        q = synth.normal_bf16((C * T, H, D), 1.0, 3, k)
        got = attention.chunk_attention(q, own_k, own_v, hist, f0, S, W, T, dtype=np.float64)
        vis = visibility.visible_frames(f0, C, S, W)
        expect = np.zeros(D)
        for f in vis:
            expect[f % D] += T
        expect /= len(vis) * T
        np.testing.assert_allclose(got[:, 0, :], np.broadcast_to(expect, (C * T, D)), atol=1e-14)


def test_gathered_keys_equal_explicit_minus_inf_mask():
    C, T, H, D, S, W = 3, 4, 2, 8, 2, 5
    ch = _rollout_inputs(6, C, T, H, D, seed=13)
    hist = _history_from(ch, C, T)
    Kall = np.concatenate([bf16.to_f32(c[1]) for c in ch])
    Vall = np.concatenate([bf16.to_f32(c[2]) for c in ch])
    frame_of_key = np.repeat(np.arange(6 * C), T)
    for k in range(6):
        f0 = k * C
        got = attention.chunk_attention(*ch[k], hist, f0, S, W, T)
        m = visibility.key_mask(f0, C, S, W, frame_of_key)
        q = bf16.to_f32(ch[k][0])
        for h in range(H):
            ref = attention.masked_attention(q[:, h], Kall[:, h], Vall[:, h], m, attention.softmax_scale(D))
            np.testing.assert_allclose(got[:, h], ref, rtol=0, atol=2e-6)
