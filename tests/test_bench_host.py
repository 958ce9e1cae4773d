"""Host-side checks of bench.py (no GPU): the one-GPU contract, the flop count behind
the roofline figure, the committed traffic summary it reads, and the CPU baseline leg
on a small workload."""

import json
import os
import subprocess
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import configs  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "GPU" in r.stderr
    assert r.stdout == ""


def test_attention_flop_count():
    # 2 flop per multiply-add, two products (Q K^T and P V), visible keys only
    cfg = configs.STEADY
    nk = (cfg.sink + cfg.window + cfg.chunk_frames) * cfg.tokens_per_frame
    assert nk == 28080
    f = bench._attn_flops(cfg.heads, cfg.head_dim, cfg.nq, nk)
    assert f == 2 * 2 * cfg.heads * cfg.head_dim * cfg.nq * nk
    assert abs(f - 8.074e11) / 8.074e11 < 1e-3


def test_traffic_summary_is_consistent():
    path = os.path.join(ROOT, "profiles", "attn_steady_traffic.json")
    with open(path) as fh:
        rec = json.load(fh)
    for key in ("source_hash", "bytes_per_launch", "kernel", "workload"):
        assert key in rec, key
    assert rec["bytes_per_launch"] > 0
    got = bench._traffic_from_profiles()
    if rec["source_hash"] == bench._kernel_source_hash():
        assert got == rec["bytes_per_launch"]
    else:   # taken on another kernel source: the bench reports no traffic
        assert got is None


def test_cpu_baseline_small_workload():
    cfg = configs.Workload(**{**configs.TOY.__dict__, "passes": 1})
    r = bench.cpu_baseline(cfg, full=False)
    assert r["kind"] == "oracle"
    assert r["unit"] == "latent frames/s per layer"
    assert r["value"] > 0 and r["seconds"] > 0 and r["cores"] >= 1
    assert "1 passes" in r["sample"]
    assert r["extrapolated"] is False and r["cpu_model"]


def test_append_bytes_count_scales_for_low_bit_caches():
    rows = 3 * 1560 * 12
    assert bench._append_bytes(rows, 128, "bf16") == 4 * rows * 128 * 2
    for kv in ("int8", "fp8", "mxfp8"):   # one code byte per value plus one 4-byte scale word per row, K and V
        assert bench._append_bytes(rows, 128, kv) == 2 * rows * 128 * 2 + 2 * rows * 128 + 2 * rows * 4
    # mxfp4: half a byte per value plus one word of four block-scale bytes per row
    assert bench._append_bytes(rows, 128, "mxfp4") == 2 * rows * 128 * 2 + 2 * rows * 64 + 2 * rows * 4


def test_stats_percentiles():
    st = bench._stats([float(x) for x in range(1, 101)])
    assert st["median"] == 50.5 and st["min"] == 1.0 and st["n"] == 100
    assert abs(st["p10"] - 10.9) < 1e-9 and abs(st["p90"] - 90.1) < 1e-9


def test_clock_sampler_reports_rather_than_raises():
    with bench.ClockSampler() as clk:
        pass
    s = clk.summary()
    assert ("median_mhz" in s) or ("error" in s)


def test_clock_sampler_keeps_fresh_tables_only(monkeypatch):
    """The metrics table refreshes about once a second: repeated reads of one table are
    one reading, idle tables are dropped, and the average power comes from the energy
    counter between the first and the last kept table."""
    import types
    state = {"reads": 0}

    def metrics(h):
        state["reads"] += 1
        k = state["reads"] // 5            # a new table every 5 reads
        busy = k >= 2                      # the first two tables are idle
        return {"firmware_timestamp": 1000 + k * 100_000_000, "current_gfxclks": [2000 + k] * 8,
                "average_gfx_activity": 100 if busy else 0, "current_socket_power": 900 + k}

    def energy(h):
        k = state["reads"] // 5
        return {"energy_accumulator": k * 1000, "counter_resolution": 1.0e6, "timestamp": 0}   # 1 kJ per table

    fake = types.SimpleNamespace(amdsmi_init=lambda: None, amdsmi_get_processor_handles=lambda: [0],
                                 amdsmi_get_gpu_metrics_info=metrics, amdsmi_get_energy_count=energy)
    monkeypatch.setitem(sys.modules, "amdsmi", fake)
    clk = bench.ClockSampler(period_s=0.001, settle_s=0.0)
    with clk:
        while state["reads"] < 40:
            time.sleep(0.001)
    s = clk.summary()
    assert s["readings"] == clk.fresh - 1 == len(clk.rows), (s, clk.fresh)   # table k = 1 is idle, k = 0 was there before
    assert s["min_mhz"] == 2002.0 and s["max_mhz"] == 2000 + s["readings"] + 1
    assert abs(s["avg_socket_w"] - 1000.0) < 1e-6        # 1 kJ per 1 s table step


def test_mfma_ceiling_library_exports_its_loop_and_checks_arguments():
    """libllceiling.so (the measured MFMA ceiling beside the roofline) is built with the
    package and rejects bad arguments before any HIP call (so this runs on the CPU)."""
    import ctypes
    import os
    import bench
    assert os.path.exists(bench.CEILING_LIB), bench.CEILING_LIB
    L = ctypes.CDLL(bench.CEILING_LIB)
    L.llc_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    buf = ctypes.create_string_buffer(16)
    assert L.llc_mfma_loop(None, 1, 1, None) != 0
    assert L.llc_mfma_loop(ctypes.addressof(buf), 0, 1, None) != 0
    assert L.llc_mfma_loop(ctypes.addressof(buf), 1, 0, None) != 0
    L.llc_mfma_loop_data.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    data = ctypes.create_string_buffer(64)
    base = (ctypes.addressof(data) + 15) // 16 * 16
    assert L.llc_mfma_loop_data(ctypes.addressof(buf), None, 1, 4, None) != 0       # no operands
    assert L.llc_mfma_loop_data(ctypes.addressof(buf), base, 1, 6, None) != 0       # iters not a multiple of 4
    assert L.llc_mfma_loop_data(ctypes.addressof(buf), base + 2, 1, 4, None) != 0   # misaligned operands
    assert L.llc_mfma_loop_data(None, base, 1, 4, None) != 0
