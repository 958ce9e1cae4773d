"""Masked softmax attention for one chunk (test infrastructure only).

Sources
-------
* dpshk.com explainer of "LongLive: Real-time Interactive Long Video
  Generation", §二 (frame-level autoregressive generation: history K/V are
  cached and reused as in a language model), §五 and §六 (the context is the
  sink frames plus the most recent window).
* wmrh.cn explainer of LongLive-2.0, §6 (the autoregressive mask: a chunk
  sees earlier chunks and itself).

What is computed
----------------
For every head h, with scale = 1/sqrt(D) evaluated once in the working
precision:

    S = (Q_h K_h^T) * scale,   S[q, j] = -inf where key j is not visible,
    P = exp(S - rowmax(S)) / rowsum(exp(S - rowmax(S))),
    O_h = P V_h.

The visible keys are those whose frame is in V(f0) (``visibility``).  Inputs
are bf16 bit patterns widened exactly; arithmetic is float32 with float32
accumulation (numpy BLAS), or float64 for the pins.
"""

import numpy as np

from . import bf16 as _bf16
from . import mxfp4 as _mx
from . import mxfp8 as _mx8
from . import quant as _quant
from . import visibility as _vis


def softmax_scale(D: int, dtype=np.float32):
    """1/sqrt(D) evaluated once in the working precision."""
    return dtype(1.0) / np.sqrt(dtype(D))


def masked_attention(Q, K, V, mask, scale, dtype=np.float32):
    """Plain masked softmax attention for one head.

    Q [nq][D], K [nk][D], V [nk][D] real arrays; ``mask`` is [nk] or [nq][nk]
    booleans (True = visible).  Every query row must see at least one key.
    Returns O [nq][D] in ``dtype``.
    """
    Q = np.asarray(Q, dtype=dtype)
    K = np.asarray(K, dtype=dtype)
    V = np.asarray(V, dtype=dtype)
    S = (Q @ K.T) * dtype(scale)
    m = np.broadcast_to(np.asarray(mask, dtype=bool), S.shape)
    if not m.any(axis=1).all():
        raise ValueError("a query row sees no key")
    S = np.where(m, S, dtype(-np.inf))
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    P = E / E.sum(axis=1, keepdims=True)
    return (P @ V).astype(dtype)


def attention_probabilities(Q, K, mask, scale, dtype=np.float64):
    """The softmax matrix P of ``masked_attention`` (used by the row-sum pin)."""
    Q = np.asarray(Q, dtype=dtype)
    K = np.asarray(K, dtype=dtype)
    S = (Q @ K.T) * dtype(scale)
    m = np.broadcast_to(np.asarray(mask, dtype=bool), S.shape)
    S = np.where(m, S, dtype(-np.inf))
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    return E / E.sum(axis=1, keepdims=True)


def attention_bruteforce_f64(Q, K, V, mask, scale):
    """Triple-loop float64 attention straight from the definition (tiny inputs)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    nq, D = Q.shape
    nk = K.shape[0]
    mask = np.broadcast_to(np.asarray(mask, dtype=bool), (nq, nk))
    out = np.zeros((nq, V.shape[1]))
    for q in range(nq):
        scores = []
        for j in range(nk):
            if mask[q, j]:
                s = 0.0
                for d in range(D):
                    s += Q[q, d] * K[j, d]
                scores.append((j, s * float(scale)))
        mx = max(s for _, s in scores)
        w = [(j, np.exp(s - mx)) for j, s in scores]
        tot = sum(e for _, e in w)
        for j, e in w:
            out[q] += (e / tot) * V[j]
    return out


def _widen(bits, dtype):
    return _bf16.to_f32(bits).astype(dtype)


def chunk_attention(Q, K_chunk, V_chunk, history, f0, S, W, tokens_per_frame,
                    kv_int8=False, rows=None, dtype=np.float32, kv=None, shot=None):
    """Attention of one chunk over V(f0), straight from the definition.

    Q, K_chunk, V_chunk: uint16 bf16 bits, shape [C*T][H][D] (own chunk).
    history(f) -> (K_f, V_f): uint16 bf16 bits [T][H][D], the K/V that frame
        f had when it entered the cache (or the recache tensor that replaced
        it).  Only frames in V(f0) are requested.
    kv: cache format "bf16" (default), "int8", "fp8", "mxfp4" or "mxfp8": for
        the low-bit formats the cached frames pass through that format's rule
        (oracle.quant: per-(token, head) absmax; oracle.mxfp4 / oracle.mxfp8:
        per block of 32 values) and are dequantised before use; own-chunk K/V
        are never quantised.  kv_int8=True is the same as kv="int8".
    rows: optional list of query rows to compute (sampled checks).
    shot: optional (Ss, fs): a shot sink of the first Ss frames of the shot that
        starts at frame fs (visibility.visible_frames_shots).
    Returns O [len(rows) or C*T][H][D] in ``dtype``.

    Keys are laid out frame by frame in ascending frame order; the mask is
    built from ``visibility.frame_mask`` over every frame [0, f0 + C), and
    only frames it marks visible contribute keys (a masked key has weight 0
    by definition, so leaving it out is the same computation).
    """
    if kv is None:
        kv = "int8" if kv_int8 else "bf16"
    if kv not in ("bf16", "int8", "fp8", "mxfp4", "mxfp8"):
        raise ValueError(f"unknown cache format {kv!r}")
    T = tokens_per_frame
    nq_all, H, D = Q.shape
    if nq_all % T:
        raise ValueError("chunk length is not a whole number of frames")
    C = nq_all // T
    Ss, fs = shot if shot is not None else (0, 0)
    fmask = _vis.frame_mask(f0, C, S, W, f0 + C, Ss, fs)
    Ks, Vs = [], []
    for f in range(f0 + C):
        if not fmask[f]:
            continue
        if f >= f0:
            a = (f - f0) * T
            Ks.append(_widen(K_chunk[a:a + T], dtype))
            Vs.append(_widen(V_chunk[a:a + T], dtype))
        else:
            kf, vf = history(f)
            if kv == "int8":
                Ks.append(_quant.dequantize(*_quant.quantize(_bf16.to_f32(kf))).astype(dtype))
                Vs.append(_quant.dequantize(*_quant.quantize(_bf16.to_f32(vf))).astype(dtype))
            elif kv == "fp8":
                Ks.append(_quant.dequantize_fp8(*_quant.quantize_fp8(_bf16.to_f32(kf))).astype(dtype))
                Vs.append(_quant.dequantize_fp8(*_quant.quantize_fp8(_bf16.to_f32(vf))).astype(dtype))
            elif kv == "mxfp4":
                Ks.append(_mx.dequantize(*_mx.quantize(_bf16.to_f32(kf))).astype(dtype))
                Vs.append(_mx.dequantize(*_mx.quantize(_bf16.to_f32(vf))).astype(dtype))
            elif kv == "mxfp8":
                Ks.append(_mx8.dequantize(*_mx8.quantize(_bf16.to_f32(kf))).astype(dtype))
                Vs.append(_mx8.dequantize(*_mx8.quantize(_bf16.to_f32(vf))).astype(dtype))
            else:
                Ks.append(_widen(kf, dtype))
                Vs.append(_widen(vf, dtype))
    Kall = np.concatenate(Ks, axis=0)
    Vall = np.concatenate(Vs, axis=0)
    Qf = _widen(Q if rows is None else Q[np.asarray(rows)], dtype)
    scale = softmax_scale(D, dtype)
    out = np.empty((Qf.shape[0], H, D), dtype=dtype)
    ones = np.ones(Kall.shape[0], dtype=bool)
    for h in range(H):
        out[:, h, :] = masked_attention(Qf[:, h, :], Kall[:, h, :], Vall[:, h, :],
                                        ones, scale, dtype)
    return out
