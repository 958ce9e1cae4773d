#!/usr/bin/env python3
"""Benchmark of the streaming sink+window KV-cache hot path on one MI355X.

One step = one steady-state chunk of a 1.3B-DiT-shaped layer: 4 denoise passes of
sink+window attention (12 heads x 128, 1560 tokens per latent frame, chunk 3,
sink 3, window 12, cache full: 28 080 visible keys) over the read-only cache, then
one append/evict of the chunk's K/V.  Inputs are seeded synthetic bf16 N(0, 0.5^2)
tensors generated on the device before the timed region (a pool of fresh Q/K/V
sets, one per pass, reused cyclically across steps).

Prints ONE JSON line with the whole-step throughput in latent frames/s per layer,
the attention kernel's roofline position, component timings (per-kernel median /
p10 / p90; int8, fp8, mxfp4 and mxfp8 caches; warm and cold appends; the 30-layer rollout, the
30-layer recache at a prompt switch and the 400-chunk int8 rollout with recache;
the shader clock read during the timed work) and the CPU oracle timed on this host
as a baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--no-components] [--no-rollouts]
                    [--workload steady|rollout|long_int8|recache|sweep|append|steady_int8|steady_fp8|
                                steady_mxfp4|steady_mxfp8|long_mxfp4|long_mxfp8]
"""

import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sink+window attention TFLOP/s & latent frames/s per layer; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
CEILING_LIB = os.path.join(ROOT, "streaming_kv_cache_block_amd", "libllceiling.so")
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
POOL = 8                       # distinct input sets cycled through the passes


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _kernel_source_hash():
    h = hashlib.sha256()
    for f in ("attn.hip", "device_common.h", "launch.h", "split_plan.h"):
        with open(os.path.join(ROOT, "streaming_kv_cache_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic_from_profiles():
    """HBM bytes per attention launch from the committed PMC summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "attn_steady_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != _kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def _attn_flops(H, D, nq, nk):
    return 4.0 * H * D * nq * nk


def _append_bytes(rows, D, kv):
    """Algorithmic bytes of writing `rows` (token, head) rows of K and V into slots: the
    bf16 inputs read, the slot codes written (2, 1 or 1/2 bytes per value for bf16,
    int8 / fp8 / mxfp8, mxfp4) and, for the low-bit caches, one 4-byte scale word per row."""
    code = {"bf16": 2 * D, "mxfp4": D // 2}.get(kv, D)
    return 2 * rows * D * 2 + 2 * rows * code + (2 * rows * 4 if kv != "bf16" else 0)


def _stats(xs):
    """mean / median / p10 / p90 / min of a list of durations (same unit)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "min": float(a.min()), "n": int(a.size)}


class ClockSampler:
    """Reads the GPU's shader clock and power with amdsmi on a background thread while
    timed work runs (context manager).  The firmware refreshes its metrics table about
    once a second, so only fresh tables count (a new firmware timestamp), and only those
    at least `settle_s` into the window with the GFX activity at >= 90%: each gives the
    mean over the 8 XCDs of the current GFX clocks and the socket power; the energy
    counter between the first and the last of them gives the average power.  Windows of
    two seconds or more give at least one reading.  summary() gives median / min / max
    in MHz and the power, or why nothing could be read."""

    def __init__(self, period_s=0.01, settle_s=0.25):
        self.period, self.settle = period_s, settle_s
        self.rows = []           # (clock MHz, socket W, energy uJ, firmware time s)
        self.fresh = 0
        self.err = None
        self._stop = threading.Event()
        self._th = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if not handles:
                raise RuntimeError("no GPU handle")
            self._smi, self._h = amdsmi, handles[0]
            self._last = self._smi.amdsmi_get_gpu_metrics_info(self._h).get("firmware_timestamp")
        except Exception as e:   # the clock is context; its absence is reported, not fatal
            self.err = f"{type(e).__name__}: {e}"

    def _loop(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
                ts = m.get("firmware_timestamp")
                if ts != self._last:
                    self._last = ts
                    self.fresh += 1
                    clks = [float(c) for c in m.get("current_gfxclks", []) if isinstance(c, (int, float))]
                    act, pw = m.get("average_gfx_activity"), m.get("current_socket_power")
                    if (clks and isinstance(act, (int, float)) and act >= 90
                            and time.perf_counter() - t0 >= self.settle):
                        e = self._smi.amdsmi_get_energy_count(self._h)
                        self.rows.append((sum(clks) / len(clks), float(pw) if isinstance(pw, (int, float)) else None,
                                          e["energy_accumulator"] * e["counter_resolution"],
                                          ts * 1e-8 if isinstance(ts, int) else None))
            except Exception as e:
                self.err = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self.err is None:
            self._th = threading.Thread(target=self._loop, daemon=True)
            self._th.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._th is not None:
            self._th.join()
        return False

    def summary(self):
        if not self.rows:
            return {"error": self.err or f"no fresh metrics table at >= 90% GFX activity ({self.fresh} fresh)"}
        import numpy as np
        clk = np.asarray([r[0] for r in self.rows])
        out = {"median_mhz": float(np.median(clk)), "min_mhz": float(clk.min()), "max_mhz": float(clk.max()),
               "readings": int(clk.size)}
        pw = [r[1] for r in self.rows if r[1] is not None]
        if pw:
            out["socket_w_median"] = float(np.median(pw))
        (e0, t0), (e1, t1) = self.rows[0][2:], self.rows[-1][2:]
        if len(self.rows) >= 2 and t0 is not None and t1 is not None and t1 > t0:
            out["avg_socket_w"] = (e1 - e0) * 1e-6 / (t1 - t0)
        out["source"] = ("amdsmi: fresh metrics tables (about 1 per second) at >= 90% GFX activity, mean of the "
                         "8 XCDs' current GFX clocks; socket power; energy counter between the first and last")
        return out


def mfma_ceiling(torch, synth=None, seconds=2.5):
    """The measured bf16 MFMA ceiling (libllceiling.so): every wave of 8 per CU (two per
    SIMD, as in the attention kernel) issues independent 32x32x16 bf16 MFMAs and nothing
    else.  Launches run back to back for about `seconds`, each timed with events on the
    launch stream; the figure is the median over the second half, once the clock has
    settled under the load (short bursts run faster than sustained work), with the shader
    clock sampled over the same launches.  With `synth`, the operands are seeded N(0, 1)
    bf16 draws, a different fragment pair in each MFMA (the matrix cores draw more power
    on such bits, so the device holds a lower clock); without, one pair of operands with
    few mantissa bits set (a best case)."""
    import ctypes
    L = ctypes.CDLL(CEILING_LIB)
    L.llc_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.llc_mfma_loop_data.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * n_cu, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    data = synth.normal_bf16_device((256 * 64,), 1.0, 977, 1) if synth is not None else None
    stream = torch.cuda.current_stream()

    def launch():
        if data is None:
            rc = L.llc_mfma_loop(out.data_ptr(), blocks, iters, stream.cuda_stream)
        else:
            rc = L.llc_mfma_loop_data(out.data_ptr(), data.data_ptr(), blocks, iters, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"MFMA ceiling launch failed ({rc})")

    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    n = 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    launch()
    e1.record(stream)
    torch.cuda.synchronize()
    n = max(20, int(seconds * 1e3 / max(e0.elapsed_time(e1), 1e-3)))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    with ClockSampler() as clk:
        for a, b in ev:
            a.record(stream)
            launch()
            b.record(stream)
        torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in ev[n // 2:]]
    ms = _stats(times)["median"]
    flop = float(blocks) * 4 * iters * 4 * 32768
    what = ("seeded N(0,1) bf16 operands, a new fragment pair per MFMA" if data is not None
            else "one operand pair with few mantissa bits set")
    return {"tflops": flop / ms / 1e9, "frac_of_nominal": flop / ms / 1e9 / PEAK_BF16_TFLOPS, "ms": ms,
            "launches": n, "sclk": clk.summary(),
            "what": "independent 32x32x16 bf16 MFMAs only, 8 waves per CU, sustained (second half of ~2.5 s); "
                    + what}


def run_steady(torch, ll, synth, cfg, steps, warmup, kv="bf16"):
    """The timed step loop (nothing but the steps between the two synchronisations),
    then as many steps again with HIP events around each launch for the per-kernel
    times; returns a dict of measurements."""
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    shape = (cfg.nq, H, D)
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    prefill = (S + W + C - 1) // C + 1
    for k in range(prefill):
        cache.append(0, synth.normal_bf16_device(shape, cfg.sigma, cfg.seed, 1, 0, k),
                     synth.normal_bf16_device(shape, cfg.sigma, cfg.seed, 2, 0, k))
    pool = [tuple(synth.normal_bf16_device(shape, cfg.sigma, cfg.seed, t, 1000 + i) for t in range(3))
            for i in range(POOL)]
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    n_vis = min(cache.frames_seen(0), S + W)
    nk = (n_vis + C) * T
    P = cfg.passes

    a0, a1 = _events(torch, steps * P), _events(torch, steps * P)
    b0, b1 = _events(torch, steps), _events(torch, steps)

    def step(i, timed):
        for p in range(P):
            q, k, v = pool[(P * i + p) % POOL]
            if timed:
                a0[i * P + p].record()
            cache.attn(0, q, k, v, out)
            if timed:
                a1[i * P + p].record()
        if timed:
            b0[i].record()
        cache.append(0, k, v)
        if timed:
            b1[i].record()

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    assert min(cache.frames_seen(0), S + W) == n_vis
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps):
        step(i, True)
    torch.cuda.synchronize()
    attn_ms = [a0[j].elapsed_time(a1[j]) for j in range(steps * P)]
    # the shader clock under this attention pass: about 2.5 seconds more of the same
    # launches (not part of any figure above) while the clock is sampled
    with ClockSampler() as clk:
        for i in range(max(1, int(2500.0 / max(sum(attn_ms) / len(attn_ms), 0.01)))):
            cache.attn(0, *pool[i % POOL], out)
        torch.cuda.synchronize()
    app_ms = [b0[i].elapsed_time(b1[i]) for i in range(steps)]
    app_bytes = _append_bytes(C * T * H, D, kv)
    attn_avg = sum(attn_ms) / len(attn_ms)
    app_avg = sum(app_ms) / len(app_ms)
    flops = _attn_flops(H, D, cfg.nq, nk)
    cache.close()
    return {
        "wall_s": wall, "keys": nk, "cached_keys": n_vis * T,
        "attn_ms": attn_avg, "attn_ms_stats": _stats(attn_ms),
        "attn_tflops": flops / attn_avg / 1e9, "attn_flops": flops,
        "append_us": app_avg * 1e3, "append_us_stats": _stats([x * 1e3 for x in app_ms]), "append_bytes": app_bytes,
        "append_gbs": app_bytes / app_avg / 1e6, "sclk": clk.summary(),
    }


def _attention_component(r):
    st = r["attn_ms_stats"]
    return {"ms": r["attn_ms"], "ms_median": st["median"], "ms_p10": st["p10"], "ms_p90": st["p90"],
            "tflops": r["attn_tflops"], "tflops_at_median": r["attn_flops"] / st["median"] / 1e9,
            "frac_mfma": r["attn_tflops"] / PEAK_BF16_TFLOPS, "keys": r["keys"], "sclk": r["sclk"]}


def _append_component(r):
    st = r["append_us_stats"]
    return {"us": r["append_us"], "us_median": st["median"], "us_p10": st["p10"], "us_p90": st["p90"],
            "gbs": r["append_gbs"], "frac_hbm": r["append_gbs"] / PEAK_HBM_GBS, "bytes": r["append_bytes"],
            "note": "HIP events around each launch inside the step (includes dispatch after the attention kernel); "
                    "the inputs were just read by the attention passes, so they are warm in the Infinity Cache"}


def run_copy_reference(torch, cfg, n=40):
    """Context for the append: the runtime's own device-to-device copy of the same bytes
    (one chunk's K and V, one launch per step like the append), issued back to back and
    timed like run_append_batch."""
    rows = cfg.nq * cfg.heads * cfg.head_dim
    src = torch.empty(2 * rows, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 1)[0], _events(torch, 1)[0]
    e0.record()
    for _ in range(n):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    byt = 2 * 2 * rows * 2
    return {"us": us, "gbs": byt / us / 1e3, "frac_hbm": byt / us / 1e3 / PEAK_HBM_GBS, "bytes": byt}


def _append_cache(torch, ll, synth, cfg, kv, W):
    C, T, H, D, S = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink
    shape = (cfg.nq, H, D)
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    pool = [tuple(synth.normal_bf16_device(shape, cfg.sigma, cfg.seed, t, 2000 + i) for t in range(2))
            for i in range(POOL)]
    for i in range((S + W + C - 1) // C + 1):
        cache.append(0, *pool[i % POOL])
    torch.cuda.synchronize()
    return cache, pool


def run_append_batch(torch, ll, synth, cfg, kv="bf16", window=None, n=40):
    """n appends of one chunk issued back to back between one pair of events: the
    kernel's own throughput, without the event bracketing of a single launch (the pool
    of 8 input chunks, 230 MB, stays partly in the Infinity Cache)."""
    W = cfg.window if window is None else window
    cache, pool = _append_cache(torch, ll, synth, cfg, kv, W)
    e0, e1 = _events(torch, 1)[0], _events(torch, 1)[0]
    e0.record()
    for i in range(n):
        cache.append(0, *pool[i % POOL])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    byt = _append_bytes(cfg.chunk_frames * cfg.tokens_per_frame * cfg.heads, cfg.head_dim, kv)
    cache.close()
    return {"us": us, "gbs": byt / us / 1e3, "frac_hbm": byt / us / 1e3 / PEAK_HBM_GBS, "bytes": byt}


def run_append_cold(torch, ll, synth, cfg, kv="bf16", window=None, n=20):
    """Appends with the caches flushed first: before each one a 1 GiB buffer is read
    (four times the 256 MB Infinity Cache, and every L2; read, so that no dirty lines
    are left to write back during the append), outside the events; each append is
    timed alone with events around its launch."""
    W = cfg.window if window is None else window
    cache, pool = _append_cache(torch, ll, synth, cfg, kv, W)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    e0, e1 = _events(torch, n), _events(torch, n)
    for i in range(n):
        flush.sum()
        e0[i].record()
        cache.append(0, *pool[i % POOL])
        e1[i].record()
    torch.cuda.synchronize()
    us = [e0[i].elapsed_time(e1[i]) * 1e3 for i in range(n)]
    st = _stats(us)
    byt = _append_bytes(cfg.chunk_frames * cfg.tokens_per_frame * cfg.heads, cfg.head_dim, kv)
    cache.close()
    del flush
    return {"us_median": st["median"], "us_p10": st["p10"], "us_p90": st["p90"], "bytes": byt,
            "gbs_at_median": byt / st["median"] / 1e3, "frac_hbm_at_median": byt / st["median"] / 1e3 / PEAK_HBM_GBS,
            "note": "Infinity Cache and L2 flushed (1 GiB read) before each append; events around the single launch"}


def run_recache_layer(torch, ll, synth, cfg, reps=10):
    """Recache of one layer at the recache workload's size, every cache format:
    projection GEMM then rewrite (two launches, K/V round trip through HBM), and the
    fused projection whose epilogue writes the slots; per-launch medians / p10 / p90."""
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    hid = cfg.hidden
    shape = (cfg.nq, H, D)
    res = {}
    for kv in ("bf16", "int8", "fp8", "mxfp4", "mxfp8"):
        cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
        for k in range(cfg.prefill_chunks):
            cache.append(0, synth.normal_bf16_device(shape, 1.0, cfg.seed, 1, k),
                         synth.normal_bf16_device(shape, 1.0, cfg.seed, 2, k))
        n = min(cache.frames_seen(0), S + W)
        h = synth.normal_bf16_device((n * T, hid), 1.0, cfg.seed, 10, 0)
        wk = synth.normal_bf16_device((hid, hid), (1.0 / hid) ** 0.5, cfg.seed, 11, 0)
        wv = synth.normal_bf16_device((hid, hid), (1.0 / hid) ** 0.5, cfg.seed, 12, 0)
        K, V = ll.kv_project(h, wk, wv)
        cache.recache(0, K, V)
        cache.recache_from_hidden(0, h, wk, wv)
        torch.cuda.synchronize()
        g0, g1, r0, r1, f0, f1 = (_events(torch, reps) for _ in range(6))
        for i in range(reps):
            g0[i].record()
            ll.kv_project(h, wk, wv, K, V)
            g1[i].record()
            r0[i].record()
            cache.recache(0, K, V)
            r1[i].record()
            f0[i].record()
            cache.recache_from_hidden(0, h, wk, wv)
            f1[i].record()
        torch.cuda.synchronize()
        gst = _stats([g0[i].elapsed_time(g1[i]) for i in range(reps)])
        rst = _stats([r0[i].elapsed_time(r1[i]) * 1e3 for i in range(reps)])
        fst = _stats([f0[i].elapsed_time(f1[i]) for i in range(reps)])
        flops = 2.0 * 2 * n * T * hid * hid
        rbytes = _append_bytes(n * T * H, D, kv)
        cache.close()
        if kv == "bf16":
            res["projection"] = {"ms": gst["mean"], "ms_median": gst["median"], "ms_p10": gst["p10"],
                                 "ms_p90": gst["p90"], "tflops": flops / gst["mean"] / 1e9,
                                 "frac_mfma": flops / gst["mean"] / 1e9 / PEAK_BF16_TFLOPS, "flop": flops}
        res[f"rewrite_{kv}"] = {"us": rst["mean"], "us_median": rst["median"], "us_p10": rst["p10"],
                                "us_p90": rst["p90"], "bytes": rbytes, "gbs": rbytes / rst["mean"] / 1e3,
                                "frac_hbm": rbytes / rst["mean"] / 1e3 / PEAK_HBM_GBS}
        res[f"fused_{kv}"] = {"ms": fst["mean"], "ms_median": fst["median"], "unfused_ms": gst["mean"] + rst["mean"] / 1e3,
                              "tflops": flops / fst["mean"] / 1e9}
    return res


def run_recache_stack(torch, ll, synth, cfg):
    """The prompt switch of the recache workload on all of its layers: a 30-layer cache
    with 6 seeded chunks appended (ring wrapped), then every layer recomputes its K/V
    from its own hidden states and weights and rewrites its 15 slots -- projection then
    rewrite, or the fused projection into the slots -- then the next chunk's attention
    on every layer.  bf16, int8 and fp8 caches; each stack timed between one pair of
    events."""
    C, T, H, D, S, W, L = (cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window,
                           cfg.layers)
    hid = cfg.hidden
    shape = (cfg.nq, H, D)
    n = min(cfg.prefill_chunks * C, S + W)
    hs = [synth.normal_bf16_device((n * T, hid), 1.0, cfg.seed, 10, l) for l in range(L)]
    ws = [(synth.normal_bf16_device((hid, hid), (1.0 / hid) ** 0.5, cfg.seed, 11, l),
           synth.normal_bf16_device((hid, hid), (1.0 / hid) ** 0.5, cfg.seed, 12, l)) for l in range(L)]
    pool = [tuple(synth.normal_bf16_device(shape, cfg.sigma, cfg.seed, t, 3000 + i) for t in range(3))
            for i in range(4)]
    K = torch.empty((n * T, H * D), dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    res = {"workload": cfg.name, "layers": L, "retained_frames": n}
    flops = 2.0 * 2 * n * T * hid * hid * L
    for kv in ("bf16", "int8", "fp8"):
        cache = ll.Cache(L, H, D, T, S, W, kv_dtype=kv)
        for l in range(L):
            for k in range(cfg.prefill_chunks):
                cache.append(l, pool[k % 4][1], pool[k % 4][2])
        torch.cuda.synchronize()
        e = _events(torch, 6)
        with ClockSampler() as clk:
            e[0].record()
            for l in range(L):
                ll.kv_project(hs[l], *ws[l], K, V)
                cache.recache(l, K, V)
            e[1].record()
            e[2].record()
            for l in range(L):
                cache.recache_from_hidden(l, hs[l], *ws[l])
            e[3].record()
            e[4].record()
            for l in range(L):
                cache.attn(l, *pool[l % 4], out)
            e[5].record()
            torch.cuda.synchronize()
        unf, fus, att = (e[2 * i].elapsed_time(e[2 * i + 1]) for i in range(3))
        res[kv] = {"stack_ms_unfused": unf, "stack_ms_fused": fus, "next_chunk_attention_ms": att,
                   "fused_tflops": flops / fus / 1e9, "rewrite_bytes": L * _append_bytes(n * T * H, D, kv),
                   "sclk": clk.summary()}
        cache.close()
    return res


def run_rollout(torch, ll, synth, cfg, kv=None):
    """Whole multi-layer rollout: per chunk, `passes` attention calls per layer, then one
    append per layer (and the recache of every layer before chunks k*recache_every).
    Inputs come from a pool of seeded device tensors made before timing.  kv: the cache
    format (default: the workload's, int8 or bf16)."""
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    shape = (cfg.nq, H, D)
    if kv is None:
        kv = "int8" if cfg.kv_int8 else "bf16"
    cache = ll.Cache(cfg.layers, H, D, T, S, W, kv_dtype=kv)
    pool = [tuple(synth.normal_bf16_device(shape, cfg.sigma, cfg.seed, t, 2000 + i) for t in range(3))
            for i in range(POOL)]
    n_re = S + W
    rec = None
    if cfg.recache_every:
        rec = (synth.normal_bf16_device((n_re * T, H, D), cfg.sigma, cfg.seed, 30),
               synth.normal_bf16_device((n_re * T, H, D), cfg.sigma, cfg.seed, 31))
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    flops = 0.0
    app_bytes = 0
    i = 0
    with ClockSampler(period_s=0.05) as clk:
        t0 = time.perf_counter()
        e0.record()
        for k in range(cfg.chunks):
            if rec is not None and k > 0 and k % cfg.recache_every == 0:
                for l in range(cfg.layers):
                    cache.recache(l, *rec)
            n_vis = min(cache.frames_seen(0), S + W)
            for p in range(cfg.passes):
                for l in range(cfg.layers):
                    q, kk, vv = pool[i % POOL]
                    i += 1
                    cache.attn(l, q, kk, vv, out)
            flops += cfg.passes * cfg.layers * _attn_flops(H, D, cfg.nq, (n_vis + C) * T)
            for l in range(cfg.layers):
                cache.append(l, kk, vv)
            app_bytes += cfg.layers * _append_bytes(C * T * H, D, kv)
            if k % 20 == 19:
                print(f"# {cfg.name}: chunk {k + 1}/{cfg.chunks}", file=sys.stderr, flush=True)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    gpu_s = e0.elapsed_time(e1) / 1e3
    frames = cfg.chunks * C
    cache.close()
    name = cfg.name if kv == ("int8" if cfg.kv_int8 else "bf16") else f"{cfg.name}, {kv} cache"
    return {"workload": name, "layers": cfg.layers, "kv": kv, "latent_frames": frames, "seconds": gpu_s,
            "wall_s": wall, "latent_frames_per_s_stack": frames / gpu_s,
            "latent_frames_per_s_per_layer": frames * cfg.layers / gpu_s, "attention_flop": flops,
            "append_bytes": app_bytes, "avg_tflops_incl_append": flops / gpu_s / 1e12,
            "recaches": (cfg.chunks - 1) // cfg.recache_every if cfg.recache_every else 0, "sclk": clk.summary()}


def run_window_sweep(torch, ll, synth, base, steps=10):
    """The pages' window/sink ablation as a kernel workload at the 1.3B shape: the
    attention pass and the append of a steady-state chunk for window 21 without sink,
    window 12 without sink and window 9 with a 3-frame sink, plus KV memory per layer."""
    res = []
    for S, W in ((0, 21), (0, 12), (3, 9)):
        cfg = configs_mod().Workload(**{**base.__dict__, "sink": S, "window": W, "name": f"sweep_s{S}_w{W}"})
        r = run_steady(torch, ll, synth, cfg, steps, 2)
        kv_bytes = 2 * (S + W) * cfg.tokens_per_frame * cfg.heads * cfg.head_dim * 2
        res.append({"sink": S, "window": W, "visible_keys": r["keys"], "attn_ms": r["attn_ms"],
                    "attn_tflops": r["attn_tflops"], "append_us": r["append_us"],
                    "step_ms": r["wall_s"] / steps * 1e3, "kv_bytes_per_layer": kv_bytes})
    ref = res[0]
    for r in res:
        r["step_time_vs_w21"] = r["step_ms"] / ref["step_ms"] - 1.0
        r["kv_memory_vs_w21"] = r["kv_bytes_per_layer"] / ref["kv_bytes_per_layer"] - 1.0
    return res


def run_appends(torch, ll, synth, cfg, n=40):
    """Appends only (for a kernel trace of the cache writes): per format, n warm appends
    back to back, then cold appends with the caches flushed in between."""
    i8w = configs_mod().LONG_INT8.window
    out = {}
    for kv, W in (("bf16", cfg.window), ("int8", i8w), ("fp8", i8w), ("mxfp4", i8w), ("mxfp8", i8w)):
        out[f"{kv}_w{W}_back_to_back"] = run_append_batch(torch, ll, synth, cfg, kv, W, n)
        out[f"{kv}_w{W}_cold"] = run_append_cold(torch, ll, synth, cfg, kv, W)
    return out


def configs_mod():
    from synth import configs
    return configs


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, full=True):
    """The CPU oracle as it stands, timed on this host.  The value: one full steady-state
    step (all passes over all 4680 query rows x 12 heads, then the append bookkeeping).
    With full=True also, each labelled: the toy workload end to end; one layer of the
    recache workload (projection and the slot-model rewrite); and the per-row cost of the
    sampled-row checks of the 30-layer rollouts, extrapolated to the whole rollouts."""
    import numpy as np
    import synth
    from oracle import attention, gemm, ring
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    configs = configs_mod()
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    shape = (cfg.nq, H, D)

    def steady_history(S, W, n_chunks, seed):
        model = ring.RingModel(S, W)
        frames = {}
        for k in range(n_chunks):
            kb = synth.normal_bf16(shape, cfg.sigma, seed, 901, k)
            vb = synth.normal_bf16(shape, cfg.sigma, seed, 902, k)
            for i in range(C):
                frames[model.f0 + i] = (kb[i * T:(i + 1) * T], vb[i * T:(i + 1) * T])
            model.append(C)
        return model, frames

    model, frames = steady_history(S, W, (S + W + C - 1) // C + 1, cfg.seed)
    inputs = [tuple(synth.normal_bf16(shape, cfg.sigma, cfg.seed, 903, t, p) for t in range(3))
              for p in range(cfg.passes)]
    t0 = time.perf_counter()
    for q, k, v in inputs:
        attention.chunk_attention(q, k, v, frames.__getitem__, model.f0, S, W, T)
    model.append(C)
    dt = time.perf_counter() - t0
    out = {"value": C / dt, "unit": "latent frames/s per layer", "cores": threads, "kind": "oracle",
           "sample": f"one full steady-state step: {cfg.passes} passes x {cfg.nq} query rows x {H} heads "
                     f"over {(min(model.f0 - C, S + W) + C) * T} keys, then the append (fp32 numpy)",
           "seconds": dt, "extrapolated": False, "cpu_model": _cpu_model()}
    if not full:
        return out
    pieces = {}
    # toy workload end to end: every pass of every chunk, append bookkeeping
    toy = configs.TOY
    tshape = (toy.nq, toy.heads, toy.head_dim)
    tm = ring.RingModel(toy.sink, toy.window)
    tframes = {}
    t0 = time.perf_counter()
    for k in range(toy.chunks):
        for p in range(toy.passes):
            q, kc, vc = (synth.normal_bf16(tshape, toy.sigma, toy.seed, t, 0, k, p) for t in range(3))
            attention.chunk_attention(q, kc, vc, tframes.__getitem__, tm.f0, toy.sink, toy.window,
                                      toy.tokens_per_frame)
        for i in range(toy.chunk_frames):
            tframes[tm.f0 + i] = (kc[i * toy.tokens_per_frame:(i + 1) * toy.tokens_per_frame],
                                  vc[i * toy.tokens_per_frame:(i + 1) * toy.tokens_per_frame])
        tm.append(toy.chunk_frames)
    pieces["toy_end_to_end"] = {"seconds": time.perf_counter() - t0, "extrapolated": False,
                                "what": f"{toy.chunks} chunks x {toy.passes} passes + appends"}
    # one layer of the recache workload: the projection (fp32 numpy) and the slot-model rewrite
    rc = configs.RECACHE
    n = min(rc.prefill_chunks * rc.chunk_frames, rc.sink + rc.window)
    h = synth.normal_bf16((n * rc.tokens_per_frame, rc.hidden), 1.0, rc.seed, 10, 0)
    wk = synth.normal_bf16((rc.hidden, rc.hidden), (1.0 / rc.hidden) ** 0.5, rc.seed, 11, 0)
    wv = synth.normal_bf16((rc.hidden, rc.hidden), (1.0 / rc.hidden) ** 0.5, rc.seed, 12, 0)
    t0 = time.perf_counter()
    gemm.project_bf16(h, wk)
    gemm.project_bf16(h, wv)
    tg = time.perf_counter() - t0
    rm = ring.RingModel(rc.sink, rc.window)
    rm.append(rc.prefill_chunks * rc.chunk_frames)
    t0 = time.perf_counter()
    rm.recache(n)
    pieces["recache_one_layer"] = {"seconds": tg + time.perf_counter() - t0, "projection_seconds": tg,
                                   "extrapolated": False,
                                   "what": f"K and V projections of {n * rc.tokens_per_frame} x {rc.hidden} hidden "
                                           f"states, then the rewrite of {n} slots in the slot model"}
    # rollouts: per-row cost of the sampled-row checks, fitted as a + b rows per
    # (chunk, pass, layer) call at the steady-state key count, extrapolated
    for name, wl in (("rollout_30_layers_extrapolated", configs.ROLLOUT),
                     ("long_int8_rollout_extrapolated", configs.LONG_INT8)):
        kv = "int8" if wl.kv_int8 else "bf16"
        m2, fr2 = steady_history(wl.sink, wl.window, (wl.sink + wl.window + C - 1) // C + 1, wl.seed)
        q, kc, vc = inputs[0]
        ts = {}
        for nrows in (16, 64):
            rows = list(range(0, cfg.nq, cfg.nq // nrows))[:nrows]
            t0 = time.perf_counter()
            attention.chunk_attention(q, kc, vc, fr2.__getitem__, m2.f0, wl.sink, wl.window, T, kv=kv, rows=rows)
            ts[nrows] = time.perf_counter() - t0
        b = max((ts[64] - ts[16]) / 48, 0.0)
        a = max(ts[16] - 16 * b, 0.0)
        per_call = a + b * cfg.nq
        calls = wl.chunks * wl.passes * wl.layers
        pieces[name] = {"seconds": per_call * calls, "extrapolated": True,
                        "per_call_seconds": per_call, "calls": calls,
                        "what": f"oracle on 16 and 64 sampled query rows at the full key count ({kv} cache), "
                                f"fitted per call and multiplied by {wl.chunks} chunks x {wl.passes} passes x "
                                f"{wl.layers} layers (early chunks see fewer keys: an overestimate); appends and "
                                f"recaches not counted"}
    out["pieces"] = pieces
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--no-rollouts", action="store_true",
                    help="leave the 30-layer rollout, the 30-layer recache and the 400-chunk int8 rollout out of "
                         "the components")
    ap.add_argument("--workload", default="steady",
                    choices=["steady", "rollout", "long_int8", "recache", "sweep", "append", "steady_int8",
                             "steady_fp8", "steady_mxfp4", "steady_mxfp8", "long_mxfp4", "long_mxfp8"],
                    help="steady (default): the one-chunk step below; the others print their own "
                         "JSON record: 30-layer rollout, 400-chunk int8 rollout with recache, "
                         "30-layer recache, window/sink sweep, appends only (warm and cold), the "
                         "steady step with an int8 / fp8 cache at window 21 (for counter runs)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="leave out the measured MFMA ceiling (about 5 s of MFMA-only launches; "
                         "for counter runs, which time every dispatch)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before the timed region, run a plain device copy of this many MiB "
                         "(reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the sink+window path runs "
              "per GPU on its own share of heads, so run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import streaming_kv_cache_block_amd as ll
    import synth
    from synth import configs

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    ll.lib()   # no fallback: fail loudly without the HIP library

    if args.calibration_copy_mib > 0:
        src = torch.empty(args.calibration_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.workload != "steady":
        if args.workload == "rollout":
            rec = run_rollout(torch, ll, synth, configs.ROLLOUT)
        elif args.workload == "long_int8":
            rec = run_rollout(torch, ll, synth, configs.LONG_INT8)
        elif args.workload in ("long_mxfp4", "long_mxfp8"):
            rec = run_rollout(torch, ll, synth, configs.LONG_INT8, kv=args.workload.split("_")[1])
        elif args.workload == "recache":
            rec = run_recache_stack(torch, ll, synth, configs.RECACHE)
        elif args.workload == "append":
            rec = {"workload": "appends", "rows": run_appends(torch, ll, synth, configs.STEADY)}
        elif args.workload in ("steady_int8", "steady_fp8", "steady_mxfp4", "steady_mxfp8"):
            kv = args.workload.split("_")[1]
            w = configs.Workload(**{**configs.STEADY.__dict__, "window": configs.LONG_INT8.window,
                                    "name": f"steady_h12_d128_t1560_s3_w21_{kv}"})
            r = run_steady(torch, ll, synth, w, args.steps, args.warmup, kv=kv)
            rec = {"workload": w.name, "attention": _attention_component(r), "append": _append_component(r)}
        else:
            rec = {"workload": "window_sink_sweep", "rows": run_window_sweep(torch, ll, synth, configs.STEADY)}
        print(json.dumps(rec), flush=True)
        return

    cfg = configs.STEADY
    r = run_steady(torch, ll, synth, cfg, args.steps, args.warmup)
    ms_per_step = r["wall_s"] / args.steps * 1e3
    value = cfg.chunk_frames * args.steps / r["wall_s"]
    ceiling = None if args.no_ceiling else mfma_ceiling(torch, synth)
    ceiling_low_bits = None if args.no_ceiling else mfma_ceiling(torch)

    components = {}
    if not args.no_components:
        i8 = configs.Workload(**{**cfg.__dict__, "window": configs.LONG_INT8.window, "kv_int8": True,
                                 "seed": configs.LONG_INT8.seed})
        ksteps = max(5, args.steps // 5)
        r8 = run_steady(torch, ll, synth, i8, ksteps, 2, kv="int8")
        rf8 = run_steady(torch, ll, synth, i8, ksteps, 2, kv="fp8")
        rm4 = run_steady(torch, ll, synth, i8, ksteps, 2, kv="mxfp4")
        rm8 = run_steady(torch, ll, synth, i8, ksteps, 2, kv="mxfp8")
        rc = run_recache_layer(torch, ll, synth, configs.RECACHE)
        components = {
            "attention_bf16": _attention_component(r),
            "append_bf16": _append_component(r),
            "append_bf16_back_to_back": run_append_batch(torch, ll, synth, cfg),
            "append_bf16_cold": run_append_cold(torch, ll, synth, cfg),
            "copy_reference_same_bytes": run_copy_reference(torch, cfg),
            "attention_int8_w21": _attention_component(r8),
            "append_int8_w21": _append_component(r8),
            "append_int8_w21_back_to_back": run_append_batch(torch, ll, synth, cfg, "int8", i8.window),
            "append_int8_w21_cold": run_append_cold(torch, ll, synth, cfg, "int8", i8.window),
            "attention_fp8_w21": _attention_component(rf8),
            "append_fp8_w21": _append_component(rf8),
            "append_fp8_w21_back_to_back": run_append_batch(torch, ll, synth, cfg, "fp8", i8.window),
            "append_fp8_w21_cold": run_append_cold(torch, ll, synth, cfg, "fp8", i8.window),
            "attention_mxfp4_w21": _attention_component(rm4),
            "append_mxfp4_w21": _append_component(rm4),
            "append_mxfp4_w21_back_to_back": run_append_batch(torch, ll, synth, cfg, "mxfp4", i8.window),
            "append_mxfp4_w21_cold": run_append_cold(torch, ll, synth, cfg, "mxfp4", i8.window),
            "attention_mxfp8_w21": _attention_component(rm8),
            "append_mxfp8_w21": _append_component(rm8),
            "append_mxfp8_w21_back_to_back": run_append_batch(torch, ll, synth, cfg, "mxfp8", i8.window),
            "append_mxfp8_w21_cold": run_append_cold(torch, ll, synth, cfg, "mxfp8", i8.window),
            "recache_layer": rc,
        }
        if not args.no_rollouts:
            print("# components: 30-layer rollout", file=sys.stderr, flush=True)
            components["rollout_30_layers_80_chunks"] = run_rollout(torch, ll, synth, configs.ROLLOUT)
            print("# components: 30-layer recache", file=sys.stderr, flush=True)
            components["recache_30_layers"] = run_recache_stack(torch, ll, synth, configs.RECACHE)
            print("# components: 400-chunk int8 rollout", file=sys.stderr, flush=True)
            components["long_int8_rollout_400_chunks"] = run_rollout(torch, ll, synth, configs.LONG_INT8)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "latent frames/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "heads": cfg.heads, "head_dim": cfg.head_dim,
                   "tokens_per_frame": cfg.tokens_per_frame, "chunk_frames": cfg.chunk_frames,
                   "sink_frames": cfg.sink, "window_frames": cfg.window, "passes_per_step": cfg.passes,
                   "query_tokens": cfg.nq, "visible_keys": r["keys"], "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": r["attn_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": r["attn_tflops"] / PEAK_BF16_TFLOPS,
                     "traffic": _traffic_from_profiles(),
                     "kernel": "attn_kernel (sink+window attention, one pass)",
                     "flop_per_launch": r["attn_flops"], "avg_launch_ms": r["attn_ms"],
                     "median_launch_ms": r["attn_ms_stats"]["median"], "sclk": r["sclk"],
                     "ceiling": ceiling, "frac_of_ceiling": r["attn_tflops"] / ceiling["tflops"] if ceiling else None,
                     "ceiling_low_bits": ceiling_low_bits},
        "attn_tflops": r["attn_tflops"],
        "components": components,
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
