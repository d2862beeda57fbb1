"""bench.py's host logic on the CPU: the CPU-baseline records (the oracle's
compute timed apart from the bf16 decode, cores from the process's CPU
affinity) and the one-GPU rule. No GPU is touched."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from relu_linear_attention_attn_amd import workloads as W  # noqa: E402


def _check_record(rec, w):
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["cores"] == len(os.sched_getaffinity(0))
    assert rec["value"] > 0 and rec["compute_s"] > 0 and rec["decode_s"] >= 0
    assert isinstance(rec["blas_threads"], int) and rec["blas_threads"] >= 1
    assert w.name in rec["sample"]


def test_cpu_baseline_forward_times_compute_only():
    w = W.custom("bench_cpu", 2, 512, 4, dtype="bf16", seed=3)
    x = W.generate(w)
    rec = bench.cpu_baseline(w, x, 0.05)
    _check_record(rec, w)
    # tokens/s = heads done x N / compute seconds / H, so compute_s alone sets it
    heads_done = rec["value"] * rec["compute_s"] * w.H / w.N
    assert abs(heads_done - round(heads_done)) < 1e-6


@pytest.mark.parametrize("fmap", ["elu1", "cos"])
def test_cpu_baseline_feature_maps(fmap):
    w = W.custom("bench_cpu_fm", 1, 256, 2, dtype="bf16", seed=4)
    _check_record(bench.cpu_baseline(w, W.generate(w), 0.02, fmap), w)


def test_cpu_baseline_backward_and_block_causal():
    w = W.custom("bench_cpu_bwd", 1, 256, 2, dtype="bf16", seed=5)
    x = W.generate(w, grad=True)
    _check_record(bench.cpu_baseline_bwd(w, x, 0.02), w)
    _check_record(bench.cpu_baseline_block_causal(w, x, 64, 0.02), w)


@pytest.mark.parametrize("fmap", ["elu1", "cos"])
def test_cpu_baseline_backward_feature_maps(fmap):
    w = W.custom("bench_cpu_bwd_fm", 1, 256, 2, dtype="bf16", seed=7)
    rec = bench.cpu_baseline_bwd(w, W.generate(w, grad=True), 0.02, fmap)
    _check_record(rec, w)
    assert fmap in rec["sample"]


def test_cpu_baseline_qkv():
    w = W.custom("bench_cpu_qkv", 1, 128, 2, dtype="bf16", seed=6)
    x = W.projection_inputs(w, 64)
    _check_record(bench.cpu_baseline_qkv(w, x, 64, 0.02), w)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
