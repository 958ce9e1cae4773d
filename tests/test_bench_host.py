"""Host-side checks of bench.py (no GPU): the one-GPU contract, the flop count behind
the roofline figure, the committed traffic summary it reads, and the CPU baseline leg
on a small workload."""

import json
import os
import subprocess
import sys

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
    r = bench.cpu_baseline(cfg)
    assert r["kind"] == "oracle"
    assert r["unit"] == "latent frames/s per layer"
    assert r["value"] > 0 and r["seconds"] > 0 and r["cores"] >= 1
    assert "1 passes" in r["sample"]
