"""GPU parity of the fused recache (projection whose epilogue writes the cache slots).

ll_cache_recache_from_hidden must leave exactly the bytes that ll_kv_project
followed by ll_cache_recache leaves (bf16 slots, int8 / fp8 codes and fp32 scales, or
MXFP4 / MXFP8 codes and block-scale words),
and those bytes must match the oracle's cache model fed the projected K/V.
Shapes: ragged token counts (T not a multiple of the 192- or 256-token tile), head_dim
64 (two heads per 128-output tile) and 128, output counts that take the 256-wide tiles
(a multiple of 256) and the 128-wide ones, a contraction of a single step, caches that
are not yet full and caches whose ring has wrapped, and the full 12-head x 128 /
1560-token / 15-frame recache.
Inputs: bf16 N(0, 1) hidden states and N(0, 1/d_in) weights from fixed seeds.
"""

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from synth import configs

from helpers import History, check_slots

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()
    return torch


def _log(msg):
    print(msg, flush=True)


def _two_caches(H, D, T, S, W, kv, appends, seed):
    a = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    b = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    hist = History(S, W, T)
    for j, n in enumerate(appends):
        kb = synth.normal_bf16((n * T, H, D), 1.0, seed, j, 0)
        vb = synth.normal_bf16((n * T, H, D), 1.0, seed, j, 1)
        for c in (a, b):
            c.append(0, synth.to_device(kb), synth.to_device(vb))
        hist.append(kb, vb)
    return a, b, hist


def _retained_equal(a, b, what):
    frames = a.slot_frames(0)
    assert frames == b.slot_frames(0)
    ga, gb = a.slot_bytes(0), b.slot_bytes(0)
    held = [i for i, f in enumerate(frames) if f >= 0]
    for key in ga:
        x, y = ga[key][held], gb[key][held]
        if x.dtype == np.float32:
            x, y = x.view(np.uint32), y.view(np.uint32)
        nbad = int(np.count_nonzero(x != y))
        assert nbad == 0, f"{what}: {key} differs in {nbad} elements"


def _case(torch, H, D, T, S, W, d_in, kv, appends, seed):
    _log(f"fused recache H={H} D={D} T={T} S={S} W={W} d_in={d_in} kv={kv} appends={appends}")
    a, b, hist = _two_caches(H, D, T, S, W, kv, appends, seed)
    n = min(hist.f0, S + W)
    h = synth.normal_bf16((n * T, d_in), 1.0, seed, 100, 0)
    wk = synth.normal_bf16((H * D, d_in), (1.0 / d_in) ** 0.5, seed, 101, 0)
    wv = synth.normal_bf16((H * D, d_in), (1.0 / d_in) ** 0.5, seed, 102, 0)
    hd, wkd, wvd = synth.to_device(h), synth.to_device(wk), synth.to_device(wv)
    K, V = ll.kv_project(hd, wkd, wvd)
    a.recache(0, K.view(n * T, H, D), V.view(n * T, H, D))
    b.recache_from_hidden(0, hd, wkd, wvd)
    _retained_equal(a, b, "fused vs project+recache")
    hist.recache(synth.to_bits(K).reshape(n * T, H, D), synth.to_bits(V).reshape(n * T, H, D))
    check_slots(b, 0, hist, kv=kv)
    return b, hist


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "mxfp4", "mxfp8"])
@pytest.mark.parametrize("H,D,T,S,W,d_in,appends", [
    (2, 64, 33, 3, 6, 128, [3, 3]),            # not full: 6 of 9 slots, ragged tiles
    (2, 64, 33, 3, 6, 192, [3, 3, 3, 3, 3]),   # wrapped ring
    (3, 128, 40, 2, 5, 256, [1, 4, 3, 2]),     # 3 heads, wrapped
    (1, 128, 7, 0, 4, 64, [2, 3]),             # no sink, tiny frames
    (4, 64, 130, 3, 0, 320, [2, 2]),           # sink only
    (2, 128, 17, 1, 3, 64, [2, 2]),            # 256 outputs (wide tiles), one 64-wide contraction step
    (1, 128, 9, 2, 2, 64, [1, 3]),             # 128 outputs, two 32-wide contraction steps
    (4, 128, 100, 2, 4, 128, [3, 3, 3]),       # 512 outputs (two wide output tiles), 600 tokens
    (6, 64, 20, 2, 3, 128, [2, 3]),            # 384 outputs of head_dim 64 (one 192 x 384 tile)
    (6, 128, 24, 1, 3, 192, [2, 2]),           # 768 outputs (two 192 x 384 tiles)
])
def test_fused_recache_matches_project_then_recache(torch_gpu, kv, H, D, T, S, W, d_in, appends):
    _case(torch_gpu, H, D, T, S, W, d_in, kv, appends, seed=300 + H * 7 + T)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "mxfp4", "mxfp8"])
def test_fused_recache_full_size(torch_gpu, kv):
    cfg = configs.RECACHE
    _case(torch_gpu, cfg.heads, cfg.head_dim, cfg.tokens_per_frame, cfg.sink, cfg.window, cfg.hidden, kv,
          [cfg.chunk_frames] * cfg.prefill_chunks, seed=cfg.seed)


def test_fused_recache_argument_errors(torch_gpu):
    torch = torch_gpu
    cache = ll.Cache(1, 2, 64, 16, 3, 6)
    h = torch.zeros((3 * 16, 128), device="cuda", dtype=torch.bfloat16)
    w = torch.zeros((128, 128), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ll.LLError) as e:        # nothing cached yet
        cache.recache_from_hidden(0, h, w, w)
    assert e.value.status == ll.LL_ERR_STATE
    cache.append(0, torch.zeros((3 * 16, 2, 64), device="cuda", dtype=torch.bfloat16),
                 torch.zeros((3 * 16, 2, 64), device="cuda", dtype=torch.bfloat16))
    with pytest.raises(ll.LLError) as e:        # wrong frame count
        cache.recache_from_hidden(0, h[:16], w, w)
    assert e.value.status == ll.LL_ERR_STATE
    h96 = torch.zeros((3 * 16, 96), device="cuda", dtype=torch.bfloat16)
    w96 = torch.zeros((128, 96), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ll.LLError) as e:        # d_in not a multiple of 64 (the library's check)
        cache.recache_from_hidden(0, h96, w96, w96)
    assert e.value.status == ll.LL_ERR_INVALID
    odd = ll.Cache(1, 1, 64, 16, 3, 6)          # heads*head_dim = 64
    odd.append(0, torch.zeros((16, 1, 64), device="cuda", dtype=torch.bfloat16),
               torch.zeros((16, 1, 64), device="cuda", dtype=torch.bfloat16))
    with pytest.raises(ll.LLError) as e:
        odd.recache_from_hidden(0, h[:16], w[:64], w[:64])
    assert e.value.status == ll.LL_ERR_INVALID
    with pytest.raises(ValueError):             # weights that do not match h: the binding's check
        cache.recache_from_hidden(0, h, w[:, :64], w[:, :64])
