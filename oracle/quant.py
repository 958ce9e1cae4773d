"""int8 KV-cache quantisation, per (token, head) row (test infrastructure only).

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
    r = np.rint((x * _F127) / safe_a[..., None])      # binary32 ops, ties to even
    r = np.clip(r, -127, 127)
    q = np.where((a == 0)[..., None], 0, r).astype(np.int8)
    return q, scale


def dequantize(q, scale):
    """(q int8 [..., D], scale float32 [...]) -> float32 [..., D]."""
    return (np.asarray(q).astype(np.float32) * np.asarray(scale, dtype=np.float32)[..., None]).astype(np.float32)
