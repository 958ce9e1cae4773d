"""Recache projection K = W_K h, V = W_V h in row form (test infrastructure only).

Sources
-------
* dpshk.com explainer of "LongLive: Real-time Interactive Long Video
  Generation", §三 item 4: the prompt enters the video tokens' hidden state
  through cross-attention, giving h'; self-attention then forms K = W_K h'
  and V = W_V h' (column form).  §三 item 5: recache re-runs this on the
  retained latents with the new prompt.

Layout used here: hidden states are rows, h [n_tokens][hidden]; the weight
is the column-form matrix W [out][in] exactly as written on the page, so
the row form of K = W_K h is K_rows = h @ W_K^T.  Bias, normalisation and
rotary position are not stated and not applied.

Arithmetic: bf16 inputs widened exactly, float32 products with float32
accumulation (numpy BLAS), result rounded to bf16 (nearest, ties to even).
"""

import numpy as np

from . import bf16 as _bf16


def project_f32(h_bits, w_bits):
    """float32 h @ W^T from bf16 bits: h [n][k], W [m][k] -> [n][m] float32."""
    h = _bf16.to_f32(h_bits)
    w = _bf16.to_f32(w_bits)
    return (h @ w.T).astype(np.float32)


def project_bf16(h_bits, w_bits):
    """K = bf16_rne(float32(h) @ float32(W)^T); returns uint16 bits [n][m]."""
    return _bf16.round_f32(project_f32(h_bits, w_bits))
