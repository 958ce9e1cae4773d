"""Pins of the MXFP4 cache rule (oracle/mxfp4.py) against the E2M1 / E8M0 format
definitions, closed forms and hand-worked cases; and of the oracle's attention over an
MXFP4 history cache (LongLive-2.0 explainer, wmrh.cn, §15.2-§15.3: a 4-bit history
cache, dequantised where it is used; the own chunk is used as given)."""

import math

import numpy as np
import pytest

import synth
from oracle import attention, bf16, mxfp4

# E2M1 magnitudes 0..7 as the format defines them (1 sign, 2 exponent bits with bias 1,
# 1 mantissa bit; exponent 0 is subnormal): listed by hand.
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_matches_format_definition():
    assert list(mxfp4.e2m1_values()) == E2M1
    codes = np.arange(16, dtype=np.uint8)
    want = [(-1.0 if c & 8 else 1.0) * E2M1[c & 7] for c in range(16)]
    got = mxfp4.e2m1_to_f64(codes)
    assert list(got) == want
    assert np.signbit(got[8])                      # code 8 is -0


def test_e2m1_rounding_midpoints_ties_to_even_and_saturation():
    # midpoint between neighbours -> the one with the even code (hand-listed)
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for y, code in ties.items():
        assert mxfp4.round_e2m1(np.float64(y)) == code, y
        assert mxfp4.round_e2m1(np.float64(-y)) == code | 8, -y
        lo, hi = np.nextafter(y, 0.0), np.nextafter(y, 10.0)
        assert mxfp4.round_e2m1(lo) == max(c for c in range(8) if E2M1[c] < y), lo
        assert mxfp4.round_e2m1(hi) == min(c for c in range(8) if E2M1[c] > y), hi
    for y in (6.0, 6.5, 7.99, 1e30):               # above the largest value: saturate
        assert mxfp4.round_e2m1(np.float64(y)) == 7
        assert mxfp4.round_e2m1(np.float64(-y)) == 15
    assert mxfp4.round_e2m1(np.float64(0.0)) == 0
    assert mxfp4.round_e2m1(np.float64(-0.0)) == 8   # the sign of zero is kept
    assert mxfp4.round_e2m1(np.float64(-0.1)) == 8
    for c in range(8):                              # every value maps to its own code
        assert mxfp4.round_e2m1(np.float64(E2M1[c])) == c


def test_e2m1_rounding_is_nearest_on_random_values():
    rng = np.random.default_rng(5)
    y = rng.uniform(-7.0, 7.0, size=20000)
    codes = mxfp4.round_e2m1(y)
    ay = np.minimum(np.abs(y), 6.0)
    got = np.abs(mxfp4.e2m1_to_f64(codes))
    dist = np.abs(np.array(E2M1)[None, :] - ay[:, None])
    assert np.all(np.abs(got - ay) <= dist.min(axis=1))          # no grid value is nearer
    assert np.all(np.signbit(mxfp4.e2m1_to_f64(codes)) == np.signbit(y))


def test_block_exponent_closed_forms():
    # e = floor(log2 a) - 2, at least -125 (a = 0 gives -125)
    cases = {1.0: -2, 1.5: -2, 1.99: -2, 2.0: -1, 6.0: 0, 7.99: 0, 8.0: 1, 0.3: -4,
             0.0: -125, 2.0 ** -130: -125, 2.0 ** -123: -125, 2.0 ** -122: -124,
             1.5 * 2.0 ** 127: 125}
    for a, e in cases.items():
        x = np.zeros(32)
        x[7] = -a
        assert mxfp4.block_exponents(x)[0] == e, a


def test_values_on_the_grid_quantise_exactly():
    rng = np.random.default_rng(6)
    n = 500
    k = rng.integers(-20, 20, size=(n, 4))
    mags = np.array(E2M1)[rng.integers(0, 8, size=(n, 4, 32))]
    mags[..., 0] = np.array([4.0, 6.0])[rng.integers(0, 2, size=(n, 4))]   # block max in [4, 8)
    x = (mags * rng.choice([-1.0, 1.0], size=mags.shape) * np.ldexp(1.0, k)[..., None]).reshape(n, 128)
    codes, e = mxfp4.quantize(x.astype(np.float32))
    assert np.array_equal(e, k)
    assert np.array_equal(mxfp4.dequantize(codes, e).astype(np.float64), x)


def test_error_bound_and_bf16_exact_dequantisation():
    x = bf16.to_f32(synth.normal_bf16((4000, 128), 1.0, 7, 0))
    codes, e = mxfp4.quantize(x)
    xh = mxfp4.dequantize(codes, e).astype(np.float64)
    assert np.array_equal(bf16.to_f32(bf16.round_f32(xh.astype(np.float32))), xh)   # bf16 values
    X = np.repeat(np.ldexp(1.0, e), 32, axis=-1)
    ay = np.abs(x.astype(np.float64)) / X
    half = np.where(ay <= 2.0, 0.25, np.where(ay <= 4.0, 0.5, 1.0))        # half the grid spacing
    bound = np.where(ay <= 6.0, half, ay - 6.0) * X
    assert np.all(np.abs(x - xh) <= bound)
    assert np.all(ay < 8.0) and np.all(ay.reshape(4000, 4, 32).max(axis=-1) >= 4.0)


def test_packing_of_codes_and_scales():
    codes = np.array([[1, 2, 3, 15, 8, 0, 7, 9]], dtype=np.uint8)
    packed = mxfp4.pack_codes(codes)
    assert list(packed[0]) == [0x21, 0xF3, 0x08, 0x97]
    assert np.array_equal(mxfp4.unpack_codes(packed), codes)
    words = mxfp4.pack_scales(np.array([[-2, 0, 125, -125]]))
    assert int(words[0]) == (125 | 127 << 8 | 252 << 16 | 2 << 24)
    assert list(mxfp4.unpack_scales(words, 4)[0]) == [-2, 0, 125, -125]
    assert int(mxfp4.pack_scales(np.array([[-1, 3]]))[0]) == (126 | 130 << 8)   # head_dim 64


def _exact_mx_history(n_rows, H, D, seed):
    """Rows whose MXFP4 quantisation is exact: each block holds grid values times 2^k with
    one entry at +-4 or +-6 times 2^k (so the block's exponent is k)."""
    rng = np.random.default_rng(seed)
    nb = D // 32
    k = rng.integers(-6, 3, size=(n_rows, H, nb))
    mags = np.array(E2M1)[rng.integers(0, 8, size=(n_rows, H, nb, 32))]
    col = rng.integers(0, 32, size=(n_rows, H, nb))
    np.put_along_axis(mags, col[..., None], np.array([4.0, 6.0])[rng.integers(0, 2, size=(n_rows, H, nb))][..., None],
                      axis=-1)
    x = (mags * rng.choice([-1.0, 1.0], size=mags.shape) * np.ldexp(1.0, k)[..., None]).reshape(n_rows, H, D)
    bits = bf16.round_f32(x.astype(np.float32))
    assert (bf16.to_f32(bits) == x).all()
    return bits


def test_mxfp4_attention_equals_bf16_when_quantisation_is_exact():
    """Exactly quantisable history rows make the MXFP4 oracle equal the bf16 one bit for
    bit, while the own chunk is generic data that quantisation would change: so the
    equality also shows the own chunk is used as given."""
    C, T, H, D, S, W = 3, 16, 2, 64, 3, 6
    n_hist = 12
    kh = _exact_mx_history(n_hist * T, H, D, 41)
    vh = _exact_mx_history(n_hist * T, H, D, 42)
    hist = lambda f: (kh[f * T:(f + 1) * T], vh[f * T:(f + 1) * T])
    for f0 in (0, 3, 9, 12):
        q, kc, vc = (synth.normal_bf16((C * T, H, D), 1.0, 43, f0, t) for t in range(3))
        assert (mxfp4.dequantize(*mxfp4.quantize(bf16.to_f32(kc))) != bf16.to_f32(kc)).any()
        a = attention.chunk_attention(q, kc, vc, hist, f0, S, W, T, kv="mxfp4")
        b = attention.chunk_attention(q, kc, vc, hist, f0, S, W, T, kv="bf16")
        assert np.array_equal(a, b), f0


def test_mxfp4_attention_worked_example():
    """One sink, one window and a one-frame own chunk, one token per frame, one head of
    32 dims (one block; scale 1/sqrt(32)).  Each history row has +-6 in a dim the query
    ignores, so its block exponent is floor(log2 6) - 2 = 0 and every other entry is
    rounded by hand to the nearest E2M1 value, ties to even:
      K: 0.3125 -> 0.5, 1.1875 -> 1.0 ; V: 2.625 -> 3.0, -3.625 -> -4.0, 5.0 -> 4.0
    (every entry is a bf16 value, so the inputs are exactly these numbers)
    The closed form equals the oracle; K or V unquantised, or the own chunk quantised,
    each move it far outside the tolerance."""
    D = 32

    def row(entries):
        r = [0.0] * D
        for d, v in entries.items():
            r[d] = v
        return r

    K_in = [row({0: 0.3125, 5: 6.0}), row({0: 1.1875, 5: -6.0})]
    K_hat = [row({0: 0.5, 5: 6.0}), row({0: 1.0, 5: -6.0})]
    V_in = [row({0: 2.625, 1: 5.0, 6: 6.0}), row({0: -3.625, 6: -6.0})]
    V_hat = [row({0: 3.0, 1: 4.0, 6: 6.0}), row({0: -4.0, 6: -6.0})]
    own_k = [row({0: 1.0, 3: 0.3125})]
    own_v = [row({0: 0.5, 1: 0.3125, 2: -0.75})]  # block max 0.75: MXFP4 would change 0.3125
    q = [row({0: 2.0})]
    as_bits = lambda rows: bf16.round_f32(np.array(rows, dtype=np.float32).reshape(len(rows), 1, D))
    kh, vh = as_bits(K_in), as_bits(V_in)
    hist = lambda f: (kh[f:f + 1], vh[f:f + 1])
    got = attention.chunk_attention(as_bits(q), as_bits(own_k), as_bits(own_v), hist, 2, 1, 1, 1,
                                    kv="mxfp4", dtype=np.float64)[0, 0]
    sc = 1.0 / math.sqrt(D)

    def closed_form(keys, vals):
        s = [sum(qi * ki for qi, ki in zip(q[0], k)) * sc for k in keys]
        e = [math.exp(x - max(s)) for x in s]
        return np.array([sum(e[j] * vals[j][d] for j in range(3)) / sum(e) for d in range(D)])

    want = closed_form(K_hat + own_k, V_hat + own_v)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # own chunk through MXFP4, by hand: own V block max 0.75 -> e = floor(log2 0.75) - 2
    # = -3, y = x * 8: 0.5 -> 4, 0.3125 -> 2.5 -> 2 (a tie, to the even code: 0.25),
    # -0.75 -> -6; own K max 1.0 -> e = -2, y = x * 4: 1.0 -> 4, 0.3125 -> 1.25 -> 1 (0.25)
    own_kq = [row({0: 1.0, 3: 0.25})]
    own_vq = [row({0: 0.5, 1: 0.25, 2: -0.75})]
    planted = {
        "K unquantised": closed_form(K_in + own_k, V_hat + own_v),
        "V unquantised": closed_form(K_hat + own_k, V_in + own_v),
        "own chunk quantised": closed_form(K_hat + own_kq, V_hat + own_vq),
    }
    for name, alt in planted.items():
        assert np.abs(alt - want).max() > 1e-4, name


# ---- MXFP8: E4M3 elements (oracle.quant's rounding, pinned against torch's
# float8_e4m3fn there) with the same power-of-two block scale ----------------------

def test_mxfp8_block_exponent_closed_forms():
    from oracle import mxfp8
    # e = floor(log2 a) - 8, at least -117 (a = 0 gives -117)
    cases = {1.0: -8, 256.0: 0, 255.5: -1, 448.0: 0, 511.0: 0, 512.0: 1, 0.3: -10,
             0.0: -117, 2.0 ** -115: -117, 2.0 ** -109: -117, 2.0 ** -108: -116,
             1.5 * 2.0 ** 127: 119}
    for a, e in cases.items():
        x = np.zeros(32)
        x[3] = a
        assert mxfp8.block_exponents(x)[0] == e, a


def test_mxfp8_grid_values_exact_saturation_and_error_bound():
    from oracle import mxfp8, quant
    rng = np.random.default_rng(8)
    vals = quant.e4m3_values()                       # 127 non-negative finite values
    n = 400
    k = rng.integers(-30, 30, size=(n, 4))
    mags = vals[rng.integers(0, 127, size=(n, 4, 32))]
    mags[..., 0] = vals[rng.integers(120, 127, size=(n, 4))]   # block max in [256, 448]
    x = (mags * rng.choice([-1.0, 1.0], size=mags.shape) * np.ldexp(1.0, k)[..., None]).reshape(n, 128)
    codes, e = mxfp8.quantize(x.astype(np.float32))
    assert np.array_equal(e, k)
    assert np.array_equal(mxfp8.dequantize(codes, e).astype(np.float64), x)
    # saturation: a block max of 480 * 2^k (a / 2^e in [256, 512)) comes back as 448 * 2^k
    y = np.zeros((1, 32))
    y[0, :3] = [480.0, -500.0, 300.0]
    c, ee = mxfp8.quantize(y.astype(np.float32))
    assert ee[0, 0] == 0 and list(mxfp8.dequantize(c, ee)[0, :3]) == [448.0, -448.0, 288.0]
    # half-step error bound on Gaussian bf16 rows, and bf16-exact dequantised values
    xg = bf16.to_f32(synth.normal_bf16((2000, 128), 1.0, 9, 0))
    cg, eg = mxfp8.quantize(xg)
    xh = mxfp8.dequantize(cg, eg).astype(np.float64)
    assert np.array_equal(bf16.to_f32(bf16.round_f32(xh.astype(np.float32))), xh)
    X = np.repeat(np.ldexp(1.0, eg), 32, axis=-1)
    ay = np.abs(xg.astype(np.float64)) / X
    # E4M3 spacing at |y| in [2^j, 2^(j+1)) is 2^(j-3) (normal), 2^-9 below 2^-6
    j = np.floor(np.log2(np.maximum(ay, 2.0 ** -6)))
    half = np.where(ay <= 448.0, 2.0 ** (j - 4), ay - 448.0)
    assert np.all(np.abs(xg - xh) <= half * X)
    # signed zero and values that round to zero keep their sign
    z = np.zeros((1, 32), dtype=np.float32)
    z[0, 0], z[0, 1], z[0, 2] = 1.0, -0.0, -2.0 ** -20
    cz, _ = mxfp8.quantize(z)
    assert cz[0, 1] == 0x80 and cz[0, 2] == 0x80 and cz[0, 3] == 0x00


def test_mxfp8_attention_equals_bf16_when_exact_and_worked_example():
    """Exactly quantisable history rows give the bf16 result bit for bit (own chunk
    generic, so it is used as given); and a hand-worked case: D = 32, one block with
    448 in a dim the query ignores (e = floor(log2 448) - 8 = 0, scale 1), entries
    rounded by hand to E4M3, ties to the even code: K 1.0625 -> 1, 1.1875 -> 1.25;
    V 3.125 -> 3, -5.25 -> -5; K or V unquantised, or the own chunk quantised, each move
    the closed form far outside the tolerance."""
    from oracle import mxfp8, quant
    C, T, H, D, S, W = 3, 16, 2, 64, 3, 6
    rng = np.random.default_rng(44)
    vals = quant.e4m3_values()

    def exact(n):
        k = rng.integers(-6, 3, size=(n, H, D // 32))
        mags = vals[rng.integers(0, 127, size=(n, H, D // 32, 32))]
        mags[..., 0] = 448.0
        x = mags * rng.choice([-1.0, 1.0], size=mags.shape) * np.ldexp(1.0, k)[..., None]
        bits = bf16.round_f32(x.reshape(n, H, D).astype(np.float32))
        assert (bf16.to_f32(bits).astype(np.float64) == x.reshape(n, H, D)).all()
        return bits

    kh, vh = exact(12 * T), exact(12 * T)
    hist = lambda f: (kh[f * T:(f + 1) * T], vh[f * T:(f + 1) * T])
    for f0 in (0, 3, 9, 12):
        q, kc, vc = (synth.normal_bf16((C * T, H, D), 1.0, 45, f0, t) for t in range(3))
        assert (mxfp8.dequantize(*mxfp8.quantize(bf16.to_f32(kc))) != bf16.to_f32(kc)).any()
        a = attention.chunk_attention(q, kc, vc, hist, f0, S, W, T, kv="mxfp8")
        b = attention.chunk_attention(q, kc, vc, hist, f0, S, W, T, kv="bf16")
        assert np.array_equal(a, b), f0

    Dw = 32

    def row(entries):
        r = [0.0] * Dw
        for d, v in entries.items():
            r[d] = v
        return r

    K_in = [row({0: 1.0625, 5: 448.0}), row({0: 1.1875, 5: -448.0})]
    K_hat = [row({0: 1.0, 5: 448.0}), row({0: 1.25, 5: -448.0})]
    V_in = [row({0: 3.125, 6: 448.0}), row({0: -5.25, 6: -448.0})]
    V_hat = [row({0: 3.0, 6: 448.0}), row({0: -5.0, 6: -448.0})]
    own_k = [row({0: 1.0})]
    own_v = [row({0: 0.5, 1: 0.3125, 2: -0.75})]   # block max 0.75: e = -9, 0.3125 * 512 = 160 exact
    own_v2 = [row({0: 0.5, 1: 0.30078125, 2: -0.75})]  # y = 154: MXFP8 would change it
    q = [row({0: 2.0})]
    as_bits = lambda rows: bf16.round_f32(np.array(rows, dtype=np.float32).reshape(len(rows), 1, Dw))
    kb, vb = as_bits(K_in), as_bits(V_in)
    hist1 = lambda f: (kb[f:f + 1], vb[f:f + 1])
    got = attention.chunk_attention(as_bits(q), as_bits(own_k), as_bits(own_v2), hist1, 2, 1, 1, 1,
                                    kv="mxfp8", dtype=np.float64)[0, 0]
    sc = 1.0 / math.sqrt(Dw)

    def closed_form(keys, vals_):
        s = [sum(qi * ki for qi, ki in zip(q[0], k)) * sc for k in keys]
        e = [math.exp(x - max(s)) for x in s]
        return np.array([sum(e[j] * vals_[j][d] for j in range(3)) / sum(e) for d in range(Dw)])

    want = closed_form(K_hat + own_k, V_hat + own_v2)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # own V through MXFP8 by hand: block max 0.75 -> e = floor(log2 0.75) - 8 = -9,
    # y = x * 512: 0.30078125 -> 154; E4M3 spacing in [128, 256) is 16, so the neighbours
    # are 144 and 160 and 154 rounds to 160 -> 160 / 512 = 0.3125
    own_vq = [row({0: 0.5, 1: 0.3125, 2: -0.75})]
    planted = {
        "K unquantised": closed_form(K_in + own_k, V_hat + own_v2),
        "V unquantised": closed_form(K_hat + own_k, V_in + own_v2),
        "own chunk quantised": closed_form(K_hat + own_k, V_hat + own_vq),
    }
    for name, alt in planted.items():
        assert np.abs(alt - want).max() > 1e-4, name
