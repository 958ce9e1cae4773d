"""int8 and fp8 (OCP E4M3) KV-cache quantisation, per (token, head) row (test
infrastructure only).

Sources
-------
* wmrh.cn explainer of LongLive-2.0, §15.2 (the history KV cache is stored
  in low precision to save memory and inter-GPU traffic) and §15.3 (it is
  dequantised before use; a slow dequantisation becomes the bottleneck).
* The symmetric int8 rule itself (one absmax per token and head, codes in
  [-127, 127]) is this library's choice for an MI355X-native low-bit cache.

Rule, written out (every operation in IEEE binary32):

    a      = max_d |x_d|                      (exact)
    scale  = a / 127                          (one correctly rounded division)
    q_d    = 0                                          if a == 0
           = clamp(rint((x_d * 127) / a), -127, 127)    otherwise
    x_hat  = float(q_d) * scale               (one rounding)

``x_d * 127`` is exact for bf16 inputs (8 + 7 significant bits < 24), so the
only roundings before ``rint`` are one division; ``rint`` rounds half to even.
Inputs are finite (precondition).

fp8 rule: the same with 448 (the largest finite E4M3 value) in place of 127 and
the E4M3 rounding of the quotient in place of ``rint``:

    scale  = a / 448,   y_d = clamp((x_d * 448) / a, -448, 448),   c_d = E4M3(y_d),
    x_hat  = value(c_d) * scale

E4M3 (OCP 8-bit floating point, "E4M3" of the OCP specification): sign bit, 4
exponent bits with bias 7, 3 mantissa bits; code 0eeeemmm has value m 2^-9 for
e = 0 and (1 + m/8) 2^(e-7) otherwise; 0x7f / 0xff are NaN, there are no
infinities, so the largest finite value is 1.75 * 2^8 = 448.  E4M3(y) is the
value nearest to |y| with ties to the even code, and the sign of y (|y| <= 448
here, so no saturation arises).  ``x_d * 448`` is exact for bf16 inputs
(448 = 7 * 2^6 adds 3 significant bits) unless it overflows binary32 (|x_d| above
about 2^119.2); then the quotient is infinite and the clamp saturates it, as the
int8 clamp does for x_d * 127.  The LongLive-2.0 explainer (§15.2) stores
the history cache in 4-bit floating point on its hardware; E4M3 with a per-row
scale is the corresponding 8-bit format native to this hardware.
"""

import numpy as np

_F127 = np.float32(127.0)


def quantize(x):
    """x: float32 [..., D] -> (q int8 [..., D], scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("quantize: inputs must be finite")
    a = np.abs(x).max(axis=-1)                       # exact
    scale = (a / _F127).astype(np.float32)           # binary32 division
    safe_a = np.where(a == 0, np.float32(1.0), a).astype(np.float32)
    with np.errstate(over="ignore"):                  # x * 127 may overflow to +-inf; the clip saturates it
        r = np.rint((x * _F127) / safe_a[..., None])  # binary32 ops, ties to even
    r = np.clip(r, -127, 127)
    q = np.where((a == 0)[..., None], 0, r).astype(np.int8)
    return q, scale


def dequantize(q, scale):
    """(q int8 [..., D], scale float32 [...]) -> float32 [..., D]."""
    return (np.asarray(q).astype(np.float32) * np.asarray(scale, dtype=np.float32)[..., None]).astype(np.float32)


_F448 = np.float32(448.0)


def e4m3_values():
    """Values of the 127 non-negative finite E4M3 codes 0..126, float64 (exact)."""
    codes = np.arange(127)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3 = e4m3_values()


def round_e4m3(y):
    """float32 y, |y| <= 448 -> uint8 E4M3 codes: nearest value, ties to the even
    code, sign bit from the sign of y (including -0)."""
    y = np.asarray(y, dtype=np.float32)
    if not (np.abs(y) <= 448).all():
        raise ValueError("round_e4m3: |y| must be <= 448")
    ay = np.abs(y).astype(np.float64)
    hi = np.searchsorted(_E4M3, ay)                  # first value >= |y|
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = ay - _E4M3[lo]
    dhi = _E4M3[hi] - ay
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    mag = np.where(take_hi, hi, lo).astype(np.uint8)
    return mag | (np.signbit(y).astype(np.uint8) << 7)


def e4m3_to_f32(codes):
    """uint8 E4M3 codes (no NaN codes) -> float32 values (exact)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = c & 0x7F
    if (mag == 0x7F).any():
        raise ValueError("e4m3_to_f32: NaN code")
    v = _E4M3[mag].astype(np.float32)
    return np.where(c & 0x80, -v, v).astype(np.float32)


def quantize_fp8(x):
    """x: float32 [..., D] -> (codes uint8 [..., D], scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("quantize_fp8: inputs must be finite")
    a = np.abs(x).max(axis=-1)                       # exact
    scale = (a / _F448).astype(np.float32)           # binary32 division
    safe_a = np.where(a == 0, np.float32(1.0), a).astype(np.float32)
    with np.errstate(over="ignore"):
        y = ((x * _F448) / safe_a[..., None]).astype(np.float32)   # binary32 ops
    codes = round_e4m3(np.clip(y, -_F448, _F448))
    codes = np.where((a == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes, scale


def dequantize_fp8(codes, scale):
    """(codes uint8 [..., D], scale float32 [...]) -> float32 [..., D]."""
    return (e4m3_to_f32(codes) * np.asarray(scale, dtype=np.float32)[..., None]).astype(np.float32)
