"""The GPU parity gates reject plausible kernel mistakes that the contract bound alone
lets through (CPU only: the mistakes are planted in oracle-computed outputs).

* Steady shape (12 heads x 128, 28 080 visible keys, N(0, 0.5^2) inputs): an output
  computed without one 20-tile piece of the split key walk stays inside max-abs 2e-2 /
  mean-abs 2e-3 but fails the scale gate (max error <= 2^-7 max|ref|).
* Peaked scores (N(0, 3^2)): values paired with the wrong key rows inside one frame, or
  the cached context's value tile taken from the wrong head, fail the rounding bound.
"""

import numpy as np
import pytest

import synth
from oracle import attention, bf16, ring
from synth import configs

from helpers import AbsHistory, History, abs_bits, compare_attention, compare_rounding_bound


def _as_gpu_bits(x):
    """An output as the kernel would return it: rounded to bf16."""
    return bf16.round_f32(np.asarray(x, dtype=np.float32))


def test_scale_gate_rejects_a_dropped_split_piece_at_the_steady_shape():
    cfg = configs.STEADY
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    shape = (cfg.nq, H, D)
    hist = History(S, W, T)
    for k in range(6):
        hist.append(synth.normal_bf16(shape, cfg.sigma, 740, 1, k), synth.normal_bf16(shape, cfg.sigma, 740, 2, k))
    q, kc, vc = (synth.normal_bf16(shape, cfg.sigma, 741, t) for t in range(3))
    rows = list(range(0, cfg.nq, 97))
    ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T, rows=rows)
    # the own chunk without keys [3392, 4672): 20 key tiles, one tail piece's worth
    keep = np.r_[0:3392, 4672:cfg.nq]
    Ks, Vs = [], []
    for f in sorted(hist.frames):
        if f < S or f >= hist.f0 - W:
            Ks.append(bf16.to_f32(hist.frames[f][0]))
            Vs.append(bf16.to_f32(hist.frames[f][1]))
    K = np.concatenate(Ks + [bf16.to_f32(kc)[keep]])
    V = np.concatenate(Vs + [bf16.to_f32(vc)[keep]])
    Qr = bf16.to_f32(q)[rows]
    planted = np.stack([attention.masked_attention(Qr[:, h], K[:, h], V[:, h], np.ones(len(K), bool),
                                                   attention.softmax_scale(D)) for h in range(H)], axis=1)
    got = _as_gpu_bits(planted)
    compare_attention(got, ref, "contract bound only")                  # passes ...
    with pytest.raises(AssertionError, match="scale gate"):
        compare_attention(got, ref, "with the scale gate", scale_gate=True)   # ... the gate does not
    compare_attention(_as_gpu_bits(ref), ref, "the oracle itself, rounded", scale_gate=True)


@pytest.mark.parametrize("mistake", ["values shifted by one token", "cache values of the next head"])
def test_rounding_bound_rejects_mispaired_values_on_peaked_scores(mistake):
    T, H, D, S, W, C = 96, 2, 64, 2, 5, 3
    shape = (C * T, H, D)
    hist = History(S, W, T)
    for k in range(4):
        hist.append(synth.normal_bf16(shape, 3.0, 750, 1, k), synth.normal_bf16(shape, 3.0, 750, 2, k))
    q, kc, vc = (synth.normal_bf16(shape, 3.0, 751, t) for t in range(3))
    ref = attention.chunk_attention(q, kc, vc, hist, hist.f0, S, W, T)
    ref_abs = attention.chunk_attention(q, kc, abs_bits(vc), AbsHistory(hist), hist.f0, S, W, T)
    compare_rounding_bound(_as_gpu_bits(ref), ref, ref_abs, "the oracle itself, rounded")

    if mistake == "values shifted by one token":
        def wrong(f):
            k, v = hist(f)
            return k, np.roll(v, 1, axis=0)
        vc_w = np.roll(vc, 1, axis=0)
    else:
        def wrong(f):
            k, v = hist(f)
            return k, np.roll(v, 1, axis=1)
        vc_w = vc
    planted = attention.chunk_attention(q, kc, vc_w, wrong, hist.f0, S, W, T)
    with pytest.raises(AssertionError):
        compare_rounding_bound(_as_gpu_bits(planted), ref, ref_abs, mistake)
