"""MXFP4 KV-cache quantisation: 4-bit E2M1 codes with one power-of-two (E8M0)
scale per block of 32 values (test infrastructure only).

Sources
-------
* wmrh.cn explainer of LongLive-2.0, §15.2 (the history KV cache is kept in
  4-bit floating point to cut memory and traffic) and §15.3 (it is dequantised
  in parallel where it is consumed).  The page uses NVIDIA's 4-bit format; the
  4-bit format native to this hardware is the OCP Microscaling (MX) one, whose
  published definition (OCP Microscaling Formats specification, v1.0: element
  format E2M1, shared scale E8M0, block size 32, scale taken from the largest
  magnitude of the block) is what this module writes out.

Element format E2M1: sign bit, 2 exponent bits with bias 1, 1 mantissa bit; no
infinities or NaN.  Magnitude code 0eem has value m/2 for e = 0 and
(1 + m/2) * 2^(e-1) otherwise: 0, 0.5, 1, 1.5, 2, 3, 4, 6.

Rule per block of 32 consecutive values x of a (token, head) row (head_dim 64:
2 blocks, 128: 4 blocks):

    a  = max |x|                                  (exact)
    e  = floor(log2 a) - 2    (2 = exponent of the largest E2M1 value, 6 = 1.5 * 2^2)
    e  = max(e, -125)         (a = 0 gives -125 too)
    y  = x / 2^e              (exact: a power of two)
    c  = sign(x) | E2M1 code nearest to min(|y|, 6), ties to the even code
    x_hat = value(c) * 2^e

The lower bound on e is this library's reading for blocks the specification
does not constrain (all zero, or a below 2^-123): with it every non-zero
dequantised value is at least 0.5 * 2^-125 = 2^-126, a normal bfloat16, so the
dequantised cache is exactly representable in bf16.  Because a / 2^e lies in
[4, 8), values above 6 * 2^e saturate to 6 * 2^e (the specification's clamp for
element formats without infinities).  A value that rounds to zero keeps its
sign (code 8 for a negative value or -0).

Storage (one cache slot row of D values): D/2 code bytes, byte k holding value
2k in its low nibble and value 2k + 1 in its high nibble; one uint32 of scale
bytes per row, byte b = e_b + 127 of block b (bytes past D/32 are 0).
"""

import numpy as np

BLOCK = 32
E_MIN = -125
E2M1_EMAX = 2


def e2m1_values():
    """Values of the 8 non-negative E2M1 magnitude codes 0..7, float64 (exact)."""
    codes = np.arange(8)
    e = codes >> 1
    m = codes & 1
    return np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * 2.0 ** (e - 1.0))


_E2M1 = e2m1_values()


def round_e2m1(y):
    """float y (any magnitude) -> uint8 E2M1 codes (0..15): the magnitude code of
    the value nearest to min(|y|, 6) with ties to the even code, sign bit 3 from
    the sign of y (including -0)."""
    y = np.asarray(y, dtype=np.float64)
    ay = np.minimum(np.abs(y), 6.0)
    hi = np.minimum(np.searchsorted(_E2M1, ay), 7)   # first value >= |y|
    lo = np.maximum(hi - 1, 0)
    dlo = ay - _E2M1[lo]
    dhi = _E2M1[hi] - ay
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    mag = np.where(take_hi, hi, lo).astype(np.uint8)
    return mag | (np.signbit(y).astype(np.uint8) << 3)


def e2m1_to_f64(codes):
    """uint8 E2M1 codes (0..15) -> float64 values (exact)."""
    c = np.asarray(codes, dtype=np.uint8)
    v = _E2M1[c & 7]
    return np.where(c & 8, -v, v)


def block_exponents(x):
    """x: float [..., n*32] -> int64 shared exponents e [..., n]."""
    x = np.asarray(x, dtype=np.float64)
    xb = x.reshape(x.shape[:-1] + (x.shape[-1] // BLOCK, BLOCK))
    a = np.abs(xb).max(axis=-1)
    _, ex = np.frexp(np.where(a == 0, 1.0, a))      # a = m 2^ex, m in [0.5, 1)
    e = (ex.astype(np.int64) - 1) - E2M1_EMAX         # floor(log2 a) - 2
    return np.where(a == 0, E_MIN, np.maximum(e, E_MIN))


def quantize(x):
    """x: float32 [..., D] (bf16 values, D a multiple of 32, D <= 128) ->
    (codes uint8 [..., D] one E2M1 code per value, exps int64 [..., D/32])."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % BLOCK or D > 4 * BLOCK:
        raise ValueError("mxfp4.quantize: head_dim must be 32, 64, 96 or 128")
    if not np.isfinite(x).all():
        raise ValueError("mxfp4.quantize: inputs must be finite")
    e = block_exponents(x)
    y = x / np.repeat(np.ldexp(1.0, e), BLOCK, axis=-1)
    return round_e2m1(y), e


def dequantize(codes, exps):
    """(codes [..., D], exps [..., D/32]) -> float32 [..., D] (exact: every value is
    a bf16 value)."""
    v = e2m1_to_f64(codes) * np.repeat(np.ldexp(1.0, np.asarray(exps)), BLOCK, axis=-1)
    return v.astype(np.float32)


def pack_codes(codes):
    """uint8 codes [..., D] -> bytes [..., D/2] (value 2k low nibble, 2k + 1 high)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    """bytes [..., D/2] -> uint8 codes [..., D]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_scales(exps):
    """int exps [..., n] (n <= 4) -> uint32 [...]: byte b = exps[b] + 127."""
    e = np.asarray(exps, dtype=np.int64)
    word = np.zeros(e.shape[:-1], dtype=np.uint64)
    for b in range(e.shape[-1]):
        word |= (e[..., b] + 127).astype(np.uint64) << np.uint64(8 * b)
    return word.astype(np.uint32)


def unpack_scales(words, n):
    """uint32 [...] -> int64 exps [..., n]."""
    w = np.asarray(words, dtype=np.uint32).astype(np.int64)
    return np.stack([((w >> (8 * b)) & 0xFF) - 127 for b in range(n)], axis=-1)
