"""Pins for oracle.quant, oracle.gemm and oracle.bf16 (CPU only)."""

from fractions import Fraction

import numpy as np
import torch

import synth
from oracle import bf16, gemm, quant


def _torch_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_including_ties():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100_000).astype(np.float32) * np.float32(3.0)
    # exact ties: upper half odd/even with lower half 0x8000
    ties = (np.arange(0, 4096, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    for arr in (x, ties, np.array([0.0, -0.0, 1e-40, -3.3e38, 3.39e38, -np.inf], dtype=np.float32)):
        assert (bf16.round_f32(arr) == _torch_bf16_bits(arr)).all()
    bits = synth.normal_bf16((1000,), 1.0, 5)
    assert (bf16.round_f32(bf16.to_f32(bits)) == bits).all()   # exact round trip


def test_quant_extremes_ties_and_zero_rows():
    row = np.array([[254.0, 1.0, 3.0, 5.0, -1.0, -3.0, -254.0, 0.0]], dtype=np.float32)
    q, s = quant.quantize(row)
    # x*127/254 = x/2: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2 (ties to even); +-absmax -> +-127
    assert q.tolist() == [[127, 0, 2, 2, 0, -2, -127, 0]]
    assert s[0] == np.float32(254.0) / np.float32(127.0) == np.float32(2.0)
    q, s = quant.quantize(np.zeros((3, 16), dtype=np.float32))
    assert (q == 0).all() and (s == 0).all()


def test_quant_matches_exact_rational_rounding_and_error_bound():
    x = bf16.to_f32(synth.normal_bf16((2000, 128), 0.5, 6))
    q, s = quant.quantize(x)
    xh = quant.dequantize(q, s)
    a = np.abs(x).max(axis=1)
    assert (np.abs(q).max(axis=1) == 127).all()          # the absmax element maps to +-127
    # |x - x_hat| <= scale/2 plus float32 rounding of q*scale and of scale itself
    err = np.abs(x - xh)
    bound = s[:, None] * np.float32(0.5) + np.abs(xh) * np.float32(2.0 ** -23) + s[:, None] * np.float32(127 * 2.0 ** -24)
    assert (err <= bound).all()
    # every code equals round-half-even of the correctly rounded binary32 quotient
    for r in range(0, 2000, 97):
        ar = Fraction(float(a[r]))
        for d in range(0, 128, 7):
            exact = Fraction(float(x[r, d])) * 127 / ar
            quot = np.float32(float(exact))          # nearest binary32 (double rounding is exact here)
            fl = int(np.floor(quot))
            frac = Fraction(float(quot)) - fl
            want = fl + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2) else 0)
            assert q[r, d] == max(-127, min(127, want))
    assert s[5] == np.float32(Fraction(float(a[5])) / 127)


def test_projection_identity_is_bit_exact():
    h = synth.normal_bf16((37, 64), 1.0, 7)
    eye = bf16.round_f32(np.eye(64, dtype=np.float32))
    assert (gemm.project_bf16(h, eye) == h).all()


def test_projection_small_integers_exact():
    rng = np.random.default_rng(2)
    hi = rng.integers(-8, 9, size=(50, 96))
    wi = rng.integers(-8, 9, size=(40, 96))
    h = bf16.round_f32(hi.astype(np.float32))
    w = bf16.round_f32(wi.astype(np.float32))
    exact = hi.astype(np.int64) @ wi.astype(np.int64).T                 # |sum| < 2^24: exact in fp32
    assert (gemm.project_f32(h, w) == exact.astype(np.float32)).all()
    assert (gemm.project_bf16(h, w) == _torch_bf16_bits(exact.astype(np.float32))).all()


def test_projection_random_within_one_bf16_ulp_of_float64():
    h = synth.normal_bf16((64, 1536), 1.0, 8)
    w = synth.normal_bf16((32, 1536), (1 / 1536) ** 0.5, 9)
    ref = bf16.to_f64(h) @ bf16.to_f64(w).T
    got = bf16.to_f64(gemm.project_bf16(h, w))
    ulp = np.abs(ref) * 2.0 ** -7 + 1e-30
    assert (np.abs(got - ref) <= ulp).all()


# ---- fp8 (OCP E4M3) rule -------------------------------------------------------

def test_e4m3_table_matches_format_definition_and_torch():
    v = quant.e4m3_values()
    assert len(v) == 127 and (np.diff(v) > 0).all()
    assert v[0] == 0 and v[1] == 2.0 ** -9 and v[7] == 7 * 2.0 ** -9     # subnormals m 2^-9
    assert v[8] == 2.0 ** -6 and v[0x7E] == 448.0 and v[0x77] == 240.0   # min normal, max, 1.875 * 2^7
    # an independent implementation of the same format: torch's float8_e4m3fn
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert (t[:127] == v).all() and np.isnan(t[127]) and np.isnan(t[255])
    assert (quant.e4m3_to_f32(np.arange(127, dtype=np.uint8) | 0x80) == -v.astype(np.float32)).all()


def _torch_e4m3(y):
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_rounding_nearest_ties_to_even_matches_torch():
    rng = np.random.default_rng(11)
    y = np.concatenate([rng.standard_normal(100_000) * 60, rng.uniform(-0.02, 0.02, 50_000),
                        rng.uniform(-448, 448, 50_000)]).astype(np.float32)
    y = np.clip(y, -448, 448)
    assert (quant.round_e4m3(y) == _torch_e4m3(y)).all()
    v = quant.e4m3_values()
    mids = (v[:-1] + v[1:]) / 2                      # exact midpoints (float32-representable)
    c = quant.round_e4m3(mids.astype(np.float32))
    assert (c % 2 == 0).all()                        # ties go to the even code
    assert (c == _torch_e4m3(mids)).all()
    assert (quant.round_e4m3(-mids.astype(np.float32)) == (c | 0x80)).all()
    # just off a midpoint goes to the nearer value
    up = np.nextafter(mids.astype(np.float32), np.float32(np.inf))
    assert (quant.e4m3_to_f32(quant.round_e4m3(up)) == v[1:].astype(np.float32)).all()
    assert quant.round_e4m3(np.float32(-0.0)) == 0x80 and quant.round_e4m3(np.float32(2.0 ** -11)) == 0


def test_fp8_quant_rule_extremes_bound_and_exact_scale():
    x = bf16.to_f32(synth.normal_bf16((1000, 128), 0.5, 12))
    c, s = quant.quantize_fp8(x)
    a = np.abs(x).max(axis=1)
    # the absmax element maps to +-448 exactly: (a * 448) / a = 448
    am = np.abs(x).argmax(axis=1)
    assert ((c[np.arange(1000), am] & 0x7F) == 0x7E).all()
    for r in range(0, 1000, 111):
        assert s[r] == np.float32(Fraction(float(a[r])) / 448)
    xh = quant.dequantize_fp8(c, s)
    y = x * np.float32(448.0) / a[:, None]
    # half an E4M3 step: 2^-4 relative in the normal range, 2^-10 absolute below 2^-6
    bound = (np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + np.abs(y) * 2.0 ** -22) * s[:, None] \
        + np.abs(xh) * 2.0 ** -23
    assert (np.abs(x - xh) <= bound).all()
    c, s = quant.quantize_fp8(np.zeros((2, 64), dtype=np.float32))
    assert (c == 0).all() and (s == 0).all()
    # fp8 keeps ~4 significant bits on every element; int8 loses small elements of a row
    xi = quant.dequantize(*quant.quantize(x))
    small = np.abs(x) < a[:, None] / 64
    assert np.abs(x - xh)[small].mean() < np.abs(x - xi)[small].mean()
