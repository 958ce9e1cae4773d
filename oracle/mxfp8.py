"""MXFP8 KV-cache quantisation: OCP E4M3 codes with one power-of-two (E8M0) scale per
block of 32 values (test infrastructure only).

Sources
-------
* wmrh.cn explainer of LongLive-2.0, §15.2 (the history KV cache is kept in low
  precision to cut memory and traffic) and §15.3 (it is dequantised in parallel
  where it is consumed).  The 8-bit member of the OCP Microscaling (MX) family
  (OCP Microscaling Formats specification, v1.0: element format E4M3, shared
  scale E8M0, block size 32, scale taken from the largest magnitude of the
  block) is written out here; the E4M3 element rounding is oracle.quant's
  (nearest value, ties to the even code, sign kept), pinned there against the
  format definition and torch's float8_e4m3fn.

Rule per block of 32 consecutive values x of a (token, head) row:

    a  = max |x|                                   (exact)
    e  = floor(log2 a) - 8     (8 = exponent of the largest E4M3 value, 448 = 1.75 * 2^8)
    e  = max(e, -117)          (a = 0 gives -117 too)
    y  = x / 2^e               (exact: a power of two)
    c  = E4M3(clamp(y, -448, 448))
    x_hat = value(c) * 2^e

The lower bound on e is this library's reading for blocks the specification does
not constrain (all zero, or a below 2^-109): with it the smallest non-zero
dequantised value is 2^-9 * 2^-117 = 2^-126, a normal bfloat16, so the
dequantised cache is exactly representable in bf16.  a / 2^e lies in [256, 512),
so values above 448 * 2^e saturate to 448 * 2^e.

Storage (one cache slot row of D values): D code bytes; one uint32 of scale bytes
per row, byte b = e_b + 127 of block b (bytes past D/32 are 0), as for MXFP4.
"""

import numpy as np

from . import quant as _quant

BLOCK = 32
E_MIN = -117
E4M3_EMAX = 8


def block_exponents(x):
    """x: float [..., n*32] -> int64 shared exponents e [..., n]."""
    x = np.asarray(x, dtype=np.float64)
    xb = x.reshape(x.shape[:-1] + (x.shape[-1] // BLOCK, BLOCK))
    a = np.abs(xb).max(axis=-1)
    _, ex = np.frexp(np.where(a == 0, 1.0, a))      # a = m 2^ex, m in [0.5, 1)
    e = (ex.astype(np.int64) - 1) - E4M3_EMAX         # floor(log2 a) - 8
    return np.where(a == 0, E_MIN, np.maximum(e, E_MIN))


def quantize(x):
    """x: float32 [..., D] (bf16 values, D a multiple of 32, D <= 128) ->
    (codes uint8 [..., D], exps int64 [..., D/32])."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % BLOCK or D > 4 * BLOCK:
        raise ValueError("mxfp8.quantize: head_dim must be 32, 64, 96 or 128")
    if not np.isfinite(x).all():
        raise ValueError("mxfp8.quantize: inputs must be finite")
    e = block_exponents(x)
    y = x / np.repeat(np.ldexp(1.0, e), BLOCK, axis=-1)          # exact
    y = np.clip(y, -448.0, 448.0).astype(np.float32)              # exact: |y| < 512, 8 significant bits
    return _quant.round_e4m3(y), e


def dequantize(codes, exps):
    """(codes [..., D], exps [..., D/32]) -> float32 [..., D] (exact bf16 values)."""
    v = _quant.e4m3_to_f32(codes).astype(np.float64) * np.repeat(np.ldexp(1.0, np.asarray(exps)), BLOCK, axis=-1)
    return v.astype(np.float32)
