#!/usr/bin/env python3
"""Benchmark of the streaming sink+window KV-cache hot path on one MI355X.

One step = one steady-state chunk of a 1.3B-DiT-shaped layer: 4 denoise passes of
sink+window attention (12 heads x 128, 1560 tokens per latent frame, chunk 3,
sink 3, window 12, cache full: 28 080 visible keys) over the read-only cache, then
one append/evict of the chunk's K/V.  Inputs are seeded synthetic bf16 N(0, 0.5^2)
tensors generated on the device before the timed region (a pool of fresh Q/K/V
sets, one per pass, reused cyclically across steps).

Prints ONE JSON line with the whole-step throughput in latent frames/s per layer,
the attention kernel's roofline position, component timings (int8 and fp8 caches,
recache projection, rewrite and the fused projection-into-slots) and the CPU oracle
timed on this host as a baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sink+window attention TFLOP/s & latent frames/s per layer; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
POOL = 8                       # distinct input sets cycled through the passes


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _kernel_source_hash():
    h = hashlib.sha256()
    for f in ("attn.hip", "device_common.h", "launch.h"):
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


def run_steady(torch, ll, synth, cfg, steps, warmup, kv_int8=False, kv=None):
    """The timed step loop (nothing but the steps between the two synchronisations),
    then as many steps again with HIP events around each launch for the per-kernel
    times; returns a dict of measurements."""
    kv = kv or ("int8" if kv_int8 else "bf16")
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
    app_ms = [b0[i].elapsed_time(b1[i]) for i in range(steps)]
    elt = 1 if kv != "bf16" else 2
    rows = C * T * H
    app_bytes = 2 * rows * D * 2 + 2 * rows * D * elt + (2 * rows * 4 if kv != "bf16" else 0)
    attn_avg = sum(attn_ms) / len(attn_ms)
    app_avg = sum(app_ms) / len(app_ms)
    flops = _attn_flops(H, D, cfg.nq, nk)
    cache.close()
    return {
        "wall_s": wall, "keys": nk, "cached_keys": n_vis * T,
        "attn_ms": attn_avg, "attn_ms_min": min(attn_ms),
        "attn_tflops": flops / attn_avg / 1e9, "attn_flops": flops,
        "append_us": app_avg * 1e3, "append_bytes": app_bytes,
        "append_gbs": app_bytes / app_avg / 1e6,
    }


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


def run_append_batch(torch, ll, synth, cfg, kv="bf16", window=None, n=40):
    """n appends of one chunk issued back to back between one pair of events: the
    kernel's own throughput, without the event bracketing of a single launch."""
    C, T, H, D, S = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink
    W = cfg.window if window is None else window
    shape = (cfg.nq, H, D)
    cache = ll.Cache(1, H, D, T, S, W, kv_dtype=kv)
    pool = [tuple(synth.normal_bf16_device(shape, cfg.sigma, cfg.seed, t, 2000 + i) for t in range(2))
            for i in range(POOL)]
    for i in range((S + W + C - 1) // C + 1):
        cache.append(0, *pool[i % POOL])
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 1)[0], _events(torch, 1)[0]
    e0.record()
    for i in range(n):
        cache.append(0, *pool[i % POOL])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    rows = C * T * H
    elt = 1 if kv != "bf16" else 2
    byt = 2 * rows * D * 2 + 2 * rows * D * elt + (2 * rows * 4 if kv != "bf16" else 0)
    cache.close()
    return {"us": us, "gbs": byt / us / 1e3, "frac_hbm": byt / us / 1e3 / PEAK_HBM_GBS, "bytes": byt}


def run_recache_layer(torch, ll, synth, cfg, reps=10):
    """Recache of one layer at the recache workload's size, bf16 and int8 caches:
    projection GEMM then rewrite (two launches, K/V round trip through HBM), and the
    fused projection whose epilogue writes the slots."""
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    hid = cfg.hidden
    shape = (cfg.nq, H, D)
    res = {}
    for kv in ("bf16", "int8", "fp8"):
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
        gms = sum(g0[i].elapsed_time(g1[i]) for i in range(reps)) / reps
        rms = sum(r0[i].elapsed_time(r1[i]) for i in range(reps)) / reps
        fms = sum(f0[i].elapsed_time(f1[i]) for i in range(reps)) / reps
        flops = 2.0 * 2 * n * T * hid * hid
        elt = 2 if kv == "bf16" else 1
        # rewrite: read bf16 K/V, write slots (+ int8 scales)
        wbytes = 2 * n * T * H * D * elt + (2 * n * T * H * 4 if kv == "int8" else 0)
        rbytes = 2 * n * T * H * D * 2 + wbytes
        cache.close()
        if kv == "bf16":
            res.update({"proj_ms": gms, "proj_tflops": flops / gms / 1e9,
                        "proj_frac": flops / gms / 1e9 / PEAK_BF16_TFLOPS,
                        "rewrite_us": rms * 1e3, "rewrite_bytes": rbytes, "rewrite_gbs": rbytes / rms / 1e6,
                        "rewrite_frac": rbytes / rms / 1e6 / PEAK_HBM_GBS})
        else:
            res.update({f"{kv}_rewrite_us": rms * 1e3, f"{kv}_rewrite_gbs": rbytes / rms / 1e6,
                        f"{kv}_rewrite_frac": rbytes / rms / 1e6 / PEAK_HBM_GBS})
        res[f"{kv}_unfused_ms"] = gms + rms
        res[f"{kv}_fused_ms"] = fms
        res[f"{kv}_fused_tflops"] = flops / fms / 1e9
    return res


def run_rollout(torch, ll, synth, cfg):
    """Whole multi-layer rollout: per chunk, `passes` attention calls per layer, then one
    append per layer (and the recache of every layer before chunks k*recache_every).
    Inputs come from a pool of seeded device tensors made before timing."""
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    shape = (cfg.nq, H, D)
    cache = ll.Cache(cfg.layers, H, D, T, S, W, kv_dtype="int8" if cfg.kv_int8 else "bf16")
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
    t0 = time.perf_counter()
    e0.record()
    i = 0
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
        if k % 20 == 19:
            print(f"# {cfg.name}: chunk {k + 1}/{cfg.chunks}", file=sys.stderr, flush=True)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = e0.elapsed_time(e1) / 1e3
    frames = cfg.chunks * C
    cache.close()
    return {"workload": cfg.name, "layers": cfg.layers, "latent_frames": frames, "seconds": gpu_s, "wall_s": wall,
            "latent_frames_per_s_stack": frames / gpu_s, "latent_frames_per_s_per_layer": frames * cfg.layers / gpu_s,
            "attention_flop": flops, "avg_tflops_incl_append": flops / gpu_s / 1e12}


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


def run_recache_stack(torch, ll, synth, cfg, reps=3):
    """Recache of every layer at a prompt switch: per layer either projection then
    rewrite, or the fused projection-into-slots (bf16 and int8 caches)."""
    r = run_recache_layer(torch, ll, synth, cfg, reps=reps)
    out = {"workload": cfg.name, "layers": cfg.layers, "per_layer": r}
    for kv in ("bf16", "int8", "fp8"):
        out[f"stack_ms_{kv}_unfused"] = cfg.layers * r[f"{kv}_unfused_ms"]
        out[f"stack_ms_{kv}_fused"] = cfg.layers * r[f"{kv}_fused_ms"]
    return out


def configs_mod():
    from synth import configs
    return configs


def cpu_baseline(cfg):
    """The CPU oracle as it stands, on one full steady-state step (4 passes over all
    4680 query rows x 12 heads, then the append bookkeeping), on this host."""
    import numpy as np  # noqa: F401
    import synth
    from oracle import attention, ring
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    C, T, H, D, S, W = cfg.chunk_frames, cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.sink, cfg.window
    shape = (cfg.nq, H, D)
    model = ring.RingModel(S, W)
    frames = {}
    prefill = (S + W + C - 1) // C + 1
    for k in range(prefill):
        kb = synth.normal_bf16(shape, cfg.sigma, cfg.seed, 901, k)
        vb = synth.normal_bf16(shape, cfg.sigma, cfg.seed, 902, k)
        for i in range(C):
            frames[model.f0 + i] = (kb[i * T:(i + 1) * T], vb[i * T:(i + 1) * T])
        model.append(C)
    inputs = [tuple(synth.normal_bf16(shape, cfg.sigma, cfg.seed, 903, t, p) for t in range(3))
              for p in range(cfg.passes)]
    t0 = time.perf_counter()
    for q, k, v in inputs:
        attention.chunk_attention(q, k, v, frames.__getitem__, model.f0, S, W, T)
    model.append(C)
    dt = time.perf_counter() - t0
    return {"value": C / dt, "unit": "latent frames/s per layer", "cores": threads, "kind": "oracle",
            "sample": f"one full steady-state step: {cfg.passes} passes x {cfg.nq} query rows x {H} heads "
                      f"over {(min(model.f0 - C, S + W) + C) * T} keys, then the append (fp32 numpy)",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--workload", default="steady", choices=["steady", "rollout", "long_int8", "recache", "sweep"],
                    help="steady (default): the one-chunk step below; the others print their own "
                         "JSON record: 30-layer rollout, 400-chunk int8 rollout with recache, "
                         "30-layer recache, window/sink sweep")
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
        elif args.workload == "recache":
            rec = run_recache_stack(torch, ll, synth, configs.RECACHE)
        else:
            rec = {"workload": "window_sink_sweep", "rows": run_window_sweep(torch, ll, synth, configs.STEADY)}
        print(json.dumps(rec), flush=True)
        return

    cfg = configs.STEADY
    r = run_steady(torch, ll, synth, cfg, args.steps, args.warmup)
    ms_per_step = r["wall_s"] / args.steps * 1e3
    value = cfg.chunk_frames * args.steps / r["wall_s"]

    components = {}
    if not args.no_components:
        i8 = configs.Workload(**{**cfg.__dict__, "window": configs.LONG_INT8.window, "kv_int8": True,
                                 "seed": configs.LONG_INT8.seed})
        r8 = run_steady(torch, ll, synth, i8, max(5, args.steps // 5), 2, kv="int8")
        rf8 = run_steady(torch, ll, synth, i8, max(5, args.steps // 5), 2, kv="fp8")
        rc = run_recache_layer(torch, ll, synth, configs.RECACHE)
        components = {
            "attention_bf16": {"ms": r["attn_ms"], "tflops": r["attn_tflops"],
                               "frac_mfma": r["attn_tflops"] / PEAK_BF16_TFLOPS, "keys": r["keys"]},
            "append_bf16": {"us": r["append_us"], "gbs": r["append_gbs"],
                            "frac_hbm": r["append_gbs"] / PEAK_HBM_GBS, "bytes": r["append_bytes"]},
            "append_bf16_back_to_back": run_append_batch(torch, ll, synth, cfg),
            "copy_reference_same_bytes": run_copy_reference(torch, cfg),
            "attention_int8_w21": {"ms": r8["attn_ms"], "tflops": r8["attn_tflops"],
                                   "frac_mfma": r8["attn_tflops"] / PEAK_BF16_TFLOPS, "keys": r8["keys"]},
            "append_int8_w21": {"us": r8["append_us"], "gbs": r8["append_gbs"],
                                "frac_hbm": r8["append_gbs"] / PEAK_HBM_GBS, "bytes": r8["append_bytes"]},
            "append_int8_w21_back_to_back": run_append_batch(torch, ll, synth, cfg, "int8", i8.window),
            "attention_fp8_w21": {"ms": rf8["attn_ms"], "tflops": rf8["attn_tflops"],
                                  "frac_mfma": rf8["attn_tflops"] / PEAK_BF16_TFLOPS, "keys": rf8["keys"]},
            "append_fp8_w21": {"us": rf8["append_us"], "gbs": rf8["append_gbs"],
                               "frac_hbm": rf8["append_gbs"] / PEAK_HBM_GBS, "bytes": rf8["append_bytes"]},
            "append_fp8_w21_back_to_back": run_append_batch(torch, ll, synth, cfg, "fp8", i8.window),
            "recache_projection": {"ms": rc["proj_ms"], "tflops": rc["proj_tflops"], "frac_mfma": rc["proj_frac"]},
            "recache_rewrite": {"us": rc["rewrite_us"], "gbs": rc["rewrite_gbs"], "frac_hbm": rc["rewrite_frac"],
                                "bytes": rc["rewrite_bytes"]},
            "recache_int8_rewrite": {"us": rc["int8_rewrite_us"], "gbs": rc["int8_rewrite_gbs"],
                                     "frac_hbm": rc["int8_rewrite_frac"]},
            "recache_fp8_rewrite": {"us": rc["fp8_rewrite_us"], "gbs": rc["fp8_rewrite_gbs"],
                                    "frac_hbm": rc["fp8_rewrite_frac"]},
            "recache_fused": {kv: {"ms": rc[f"{kv}_fused_ms"], "unfused_ms": rc[f"{kv}_unfused_ms"],
                                   "tflops": rc[f"{kv}_fused_tflops"]} for kv in ("bf16", "int8", "fp8")},
        }

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
                     "flop_per_launch": r["attn_flops"], "avg_launch_ms": r["attn_ms"]},
        "attn_tflops": r["attn_tflops"],
        "components": components,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
