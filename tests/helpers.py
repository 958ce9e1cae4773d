"""Shared helpers of the GPU parity tests: history bookkeeping, comparisons, row samples.

The history kept here is plain input bookkeeping (which bytes the caller passed for
which frame); what a chunk may see is decided by the oracle alone.
"""

import numpy as np

import synth
from oracle import bf16, quant, ring

# attention acceptance bounds against the fp32 oracle (same bf16-rounded inputs)
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


class History:
    """frame id -> (K bits, V bits) [T][H][D] uint16, as last written by the caller.

    Append stores each new frame's input bytes; recache replaces the retained
    frames' entries with the recache tensors' blocks (the oracle's recache rule
    decides which frame each block belongs to).
    """

    def __init__(self, S, W, T, Ss=0):
        self.T = T
        self.frames = {}
        self.model = ring.RingModel(S, W, Ss)

    def begin_shot(self):
        self.model.begin_shot()

    @property
    def shot(self):
        """(Ss, fs) for the oracle's chunk_attention."""
        return (self.model.Ss, self.model.fs)

    def append(self, K_bits, V_bits):
        n = K_bits.shape[0] // self.T
        f0 = self.model.f0
        for i in range(n):
            self.frames[f0 + i] = (K_bits[i * self.T:(i + 1) * self.T], V_bits[i * self.T:(i + 1) * self.T])
        self.model.append(n, src_of_frame=lambda f: f)

    def recache(self, K_bits, V_bits):
        retained = self.model.retained_frames()
        for idx, f in enumerate(retained):
            self.frames[f] = (K_bits[idx * self.T:(idx + 1) * self.T], V_bits[idx * self.T:(idx + 1) * self.T])
        self.model.recache(len(retained))

    def recache_window(self, K_bits, V_bits):
        m = self.model
        window = list(range(max(m.S, m.f0 - m.W), m.f0))
        for idx, f in enumerate(window):
            self.frames[f] = (K_bits[idx * self.T:(idx + 1) * self.T], V_bits[idx * self.T:(idx + 1) * self.T])

    def __call__(self, f):
        return self.frames[f]

    @property
    def f0(self):
        return self.model.f0


def compare_attention(gpu_out, ref, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    """gpu_out: torch bf16 (or uint16 bits); ref: float array of the same shape."""
    got = bf16.to_f32(gpu_out if isinstance(gpu_out, np.ndarray) else synth.to_bits(gpu_out))
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    mx, mn = float(err.max()), float(err.mean())
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3g} mean-abs {mn:.3g}"
    return mx, mn


def check_slots(cache, layer, hist, kv_int8=False, kv=None):
    """Slot->frame map equals the slot model; every occupied slot holds exactly the
    bytes (or the int8 / fp8 quantisation) of the frame it claims; the occupied frames
    are the cached part of the visible set."""
    if kv is None:
        kv = "int8" if kv_int8 else "bf16"
    sf = cache.slot_frames(layer)
    assert sf == hist.model.slot_frame, (sf, hist.model.slot_frame)
    assert cache.frames_seen(layer) == hist.f0
    got = cache.slot_bytes(layer)
    for s, f in enumerate(sf):
        if f < 0:
            continue
        kb, vb = hist(f)
        if kv == "bf16":
            assert np.array_equal(got["K"][s].view(np.uint16), kb), f"K slot {s} frame {f}"
            assert np.array_equal(got["V"][s].view(np.uint16), vb), f"V slot {s} frame {f}"
        else:
            for name, src in (("K", kb), ("V", vb)):
                if kv == "int8":
                    q, sc = quant.quantize(bf16.to_f32(src))
                    same = got[name][s].view(np.int8) == q
                else:
                    q, sc = quant.quantize_fp8(bf16.to_f32(src))
                    same = got[name][s].view(np.uint8) == q
                if not same.all():
                    bad = np.argwhere(~same)[:4].tolist()
                    raise AssertionError(f"{name} codes slot {s} frame {f}: {int((~same).sum())} differ, e.g. {bad}")
                assert np.array_equal(got[name + "_scale"][s].view(np.uint32), sc.view(np.uint32)), \
                    f"{name} scales slot {s} frame {f}"


def sample_rows(nq, T, seed, n_random=32):
    fixed = [0, 1, T - 1, T, 2 * T - 1, 2 * T, 3 * T - 1, 31, 32, 63, 64, 127, 128, 255, 256,
             4607, 4608, nq - 1]
    rng = np.random.default_rng(seed)
    rows = set(r for r in fixed if 0 <= r < nq) | set(int(x) for x in rng.integers(0, nq, n_random))
    return sorted(rows)
