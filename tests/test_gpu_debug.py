"""The debug library (host side built with LL_DEBUG) on the GPU.

Every slot of a fresh debug cache is poisoned (bf16 NaN, NaN scales for int8 / fp8,
E8M0 NaN block-scale bytes 0xFF for MXFP4 / MXFP8)
and the slots a recache rewrites are poisoned again just before.  So:
  * a toy rollout through the debug library gives finite outputs, byte for byte the
    normal library's: attention never read a slot no frame was written to;
  * after a recache, a window-only recache and a fused projection into the slots, no
    retained slot holds poison: the rewrite reached every slot it owns (the window-only
    recache left the sink as it was, not poisoned), and the fused rewrite's bytes are
    the normal library's.
"""

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from oracle import bf16
from synth import configs

from helpers import History, check_slots

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()
    ll.lib(debug=True)
    return torch


def _poisoned(got, kv):
    """Per slot: True where any K or V value of the slot dequantises to NaN."""
    if kv == "bf16":
        k = np.isnan(bf16.to_f32(got["K"].view(np.uint16))).reshape(got["K"].shape[0], -1).any(axis=1)
        v = np.isnan(bf16.to_f32(got["V"].view(np.uint16))).reshape(got["V"].shape[0], -1).any(axis=1)
    elif kv in ("mxfp4", "mxfp8"):   # a written block scale byte is e + 127 <= 252; 0xFF is E8M0's NaN
        k = (got["K_scale"].view(np.uint8) == 0xFF).reshape(got["K_scale"].shape[0], -1).any(axis=1)
        v = (got["V_scale"].view(np.uint8) == 0xFF).reshape(got["V_scale"].shape[0], -1).any(axis=1)
    else:
        k = np.isnan(got["K_scale"]).reshape(got["K_scale"].shape[0], -1).any(axis=1)
        v = np.isnan(got["V_scale"]).reshape(got["V_scale"].shape[0], -1).any(axis=1)
    return k | v


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "mxfp4", "mxfp8"])
def test_debug_library_poisons_and_matches(torch_gpu, kv):
    cfg = configs.TOY
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    dbg = ll.Cache(1, H, D, T, S, W, kv_dtype=kv, debug=True)
    ref = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    assert _poisoned(dbg.slot_bytes(0), kv).all(), "a fresh debug cache is poisoned everywhere"
    hist = History(S, W, T)
    shape = (cfg.nq, H, D)
    for k in range(cfg.chunks):
        for p in range(cfg.passes):
            q, kc, vc = (synth.to_device(synth.normal_bf16(shape, cfg.sigma, 770, t, k, p)) for t in range(3))
            a = dbg.attn(0, q, kc, vc)
            b = ref.attn(0, q, kc, vc)
            got = synth.to_bits(a)
            assert np.isfinite(bf16.to_f32(got)).all(), f"chunk {k}: attention read a poisoned slot"
            assert np.array_equal(got, synth.to_bits(b)), f"chunk {k}: debug and normal libraries differ"
        dbg.append(0, kc, vc)
        ref.append(0, kc, vc)
        hist.append(synth.to_bits(kc), synth.to_bits(vc))
        poisoned = _poisoned(dbg.slot_bytes(0), kv)
        occupied = np.array([f >= 0 for f in dbg.slot_frames(0)])
        assert not poisoned[occupied].any() and poisoned[~occupied].all(), (k, poisoned, occupied)
    check_slots(dbg, 0, hist, kv=kv)
    # recache: every retained slot is poisoned first, then rewritten
    n = len(hist.model.retained_frames())
    K_all, V_all = (synth.normal_bf16((n * T, H, D), 1.0, 771, t) for t in range(2))
    dbg.recache(0, synth.to_device(K_all), synth.to_device(V_all))
    hist.recache(K_all, V_all)
    assert not _poisoned(dbg.slot_bytes(0), kv).any()
    check_slots(dbg, 0, hist, kv=kv)
    # window-only recache: the window slots are poisoned and rewritten, the sink is kept
    nw = len(hist.model.window_frames())
    K_w, V_w = (synth.normal_bf16((nw * T, H, D), 1.0, 772, t) for t in range(2))
    dbg.recache_window(0, synth.to_device(K_w), synth.to_device(V_w))
    hist.recache_window(K_w, V_w)
    assert not _poisoned(dbg.slot_bytes(0), kv).any()
    check_slots(dbg, 0, hist, kv=kv)
    # fused projection into the slots: poisoned first, then every retained slot written,
    # byte for byte what the normal library writes
    d_in = 128
    n = len(hist.model.retained_frames())
    h = synth.to_device(synth.normal_bf16((n * T, d_in), 1.0, 773, 0))
    w_k = synth.to_device(synth.normal_bf16((H * D, d_in), 0.05, 773, 1))
    w_v = synth.to_device(synth.normal_bf16((H * D, d_in), 0.05, 773, 2))
    dbg.recache_from_hidden(0, h, w_k, w_v)
    ref.recache_from_hidden(0, h, w_k, w_v)
    got, want = dbg.slot_bytes(0), ref.slot_bytes(0)
    assert not _poisoned(got, kv).any()
    for name in got:
        assert np.array_equal(got[name].view(np.uint8), want[name].view(np.uint8)), name
    dbg.close()
    ref.close()
