"""GPU parity of the long streaming rollouts at full size, on sampled outputs.

* 30-layer rollout: 80 chunks (240 latent frames), sink 3, window 12, 4 denoise
  passes per chunk with fresh bf16 N(0, 0.5^2) inputs per pass (seed 2).
* Long int8 rollout: 400 chunks (1200 latent frames), 30 layers, window 21, int8
  cache, a recache of every layer's retained cache before chunks 50, 100, ..., 350
  with fresh seeded tensors (seed 4).

Both run every layer; layers 0, 15 and 29 are checked against the oracle.

Inputs come from the seeded device generator; any frame the oracle asks for is
regenerated on the device from its key and downloaded (the first one is also
regenerated on the host by the generator's twin and must match), so no history is
stored.  Checked: slot ->
frame maps of every run layer after every append (bit-exact), sampled query rows
(tile edges, frame edges, random) against the oracle over every key the oracle deems
visible, full slot bytes at a few chunks and after each recache.
"""

import time
from collections import OrderedDict

import numpy as np
import pytest

import streaming_kv_cache_block_amd as ll
import synth
from oracle import attention, ring
from synth import configs

from helpers import check_slots, compare_attention, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ll.lib()
    return torch


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


class RegenHistory:
    """frame -> bf16 bits of the K/V it holds, regenerated from the seeded generator.

    Appended frames come from the last denoise pass of their chunk; a recache replaces
    the retained frames (the oracle's recache order decides which block goes where).
    """

    def __init__(self, cfg, layer):
        self.cfg, self.layer = cfg, layer
        self.model = ring.RingModel(cfg.sink, cfg.window)
        self.src = {}                     # frame -> ("chunk", k) | ("recache", r, idx)
        self.lru = OrderedDict()
        self.twin_checked = False

    def _fetch(self, key, shape):
        if key not in self.lru:
            kb = synth.to_bits(synth.normal_bf16_device(shape, self.cfg.sigma, *key[0]))
            vb = synth.to_bits(synth.normal_bf16_device(shape, self.cfg.sigma, *key[1]))
            if not self.twin_checked:
                # the device draw is the host generator's, bit for bit (synth.philox)
                assert np.array_equal(kb, synth.normal_bf16_philox(shape, self.cfg.sigma, *key[0]))
                self.twin_checked = True
            self.lru[key] = (kb, vb)
            while len(self.lru) > 12:
                self.lru.popitem(last=False)
        return self.lru[key]

    def append_chunk(self, k):
        C = self.cfg.chunk_frames
        for i in range(C):
            self.src[self.model.f0 + i] = ("chunk", k)
        self.model.append(C)

    def recache(self, r):
        for idx, f in enumerate(self.model.retained_frames()):
            self.src[f] = ("recache", r, idx)
        self.model.recache(len(self.model.retained_frames()))

    def __call__(self, f):
        cfg, T = self.cfg, self.cfg.tokens_per_frame
        s = self.src[f]
        if s[0] == "chunk":
            k = s[1]
            kb, vb = self._fetch((chunk_key(cfg, 1, self.layer, k, cfg.passes - 1),
                                  chunk_key(cfg, 2, self.layer, k, cfg.passes - 1)),
                                 (cfg.nq, cfg.heads, cfg.head_dim))
            r = f - k * cfg.chunk_frames
        else:
            _, rr, idx = s
            n = cfg.sink + cfg.window
            kb, vb = self._fetch((recache_key(cfg, 1, self.layer, rr), recache_key(cfg, 2, self.layer, rr)),
                                 (n * T, cfg.heads, cfg.head_dim))
            r = idx
        return kb[r * T:(r + 1) * T], vb[r * T:(r + 1) * T]

    @property
    def f0(self):
        return self.model.f0


def chunk_key(cfg, tensor, layer, k, p):
    return (cfg.seed, tensor, layer, k, p)


def recache_key(cfg, tensor, layer, r):
    return (cfg.seed, 10 + tensor, layer, r)


def _rollout(torch, cfg, layers, check_layers, check_chunks, slot_chunks):
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    shape = (cfg.nq, H, D)
    cache = ll.Cache(len(layers), H, D, T, S, W, kv_dtype="int8" if cfg.kv_int8 else "bf16")
    hist = {l: RegenHistory(cfg, l) for l in layers}
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    rows = sample_rows(cfg.nq, T, seed=cfg.seed, n_random=16)
    n_checks, worst = 0, 0.0
    t0 = time.time()
    for k in range(cfg.chunks):
        if cfg.recache_every and k > 0 and k % cfg.recache_every == 0:
            r = k // cfg.recache_every
            n = min(hist[layers[0]].f0, S + W)
            for li, l in enumerate(layers):
                K_all = synth.normal_bf16_device((n * T, H, D), cfg.sigma, *recache_key(cfg, 1, l, r))
                V_all = synth.normal_bf16_device((n * T, H, D), cfg.sigma, *recache_key(cfg, 2, l, r))
                cache.recache(li, K_all, V_all)
                hist[l].recache(r)
                if l in check_layers:
                    check_slots(cache, li, hist[l], kv_int8=cfg.kv_int8)
            _log(f"{cfg.name}: recache before chunk {k} checked")
        last = {}
        for p in range(cfg.passes):
            for li, l in enumerate(layers):
                q = synth.normal_bf16_device(shape, cfg.sigma, *chunk_key(cfg, 0, l, k, p))
                kc = synth.normal_bf16_device(shape, cfg.sigma, *chunk_key(cfg, 1, l, k, p))
                vc = synth.normal_bf16_device(shape, cfg.sigma, *chunk_key(cfg, 2, l, k, p))
                cache.attn(li, q, kc, vc, out)
                if l in check_layers and k in check_chunks and p in (0, cfg.passes - 1):
                    qb, kb, vb = synth.to_bits(q), synth.to_bits(kc), synth.to_bits(vc)
                    ref = attention.chunk_attention(qb, kb, vb, hist[l], hist[l].f0, S, W, T,
                                                    kv_int8=cfg.kv_int8, rows=rows)
                    mx, _ = compare_attention(synth.to_bits(out)[rows], ref, f"layer {l} chunk {k} pass {p}",
                                              scale_gate=True)
                    worst = max(worst, mx)
                    n_checks += 1
                if p == cfg.passes - 1:
                    last[l] = (kc, vc)
        for li, l in enumerate(layers):
            cache.append(li, *last[l])
            hist[l].append_chunk(k)
            assert cache.slot_frames(li) == hist[l].model.slot_frame, (l, k)
            if l in check_layers and k in slot_chunks:
                check_slots(cache, li, hist[l], kv_int8=cfg.kv_int8)
        if k % 20 == 0 or k == cfg.chunks - 1:
            _log(f"{cfg.name}: chunk {k} done, {n_checks} sampled checks, worst max-abs {worst:.2e}, "
                 f"{time.time() - t0:.1f}s")
    cache.close()
    return n_checks


def test_rollout_30_layers_80_chunks(torch_gpu):
    cfg = configs.ROLLOUT
    wrap = cfg.window // cfg.chunk_frames
    check_chunks = {0, 1, 2, 3, 4, 5, 6, 9, 10, 40, cfg.chunks - 1} | {5 + wrap * i for i in range(3)}
    n = _rollout(torch_gpu, cfg, list(range(cfg.layers)), {0, 15, cfg.layers - 1}, check_chunks,
                 {4, 5, 6, cfg.chunks - 1})
    assert n >= 30


def test_long_int8_rollout_with_recache(torch_gpu):
    cfg = configs.LONG_INT8
    check_chunks = {0, 1, 2, 7, 8, 9, 49, 50, 51, 100, 101, cfg.chunks - 1}
    n = _rollout(torch_gpu, cfg, list(range(cfg.layers)), {0, 15, cfg.layers - 1}, check_chunks,
                 {7, 8, cfg.chunks - 1})
    assert n >= 30
