"""bench.py's command-line contract on the host (no GPU): one GPU only, no
CPU fallback, and the HBM traffic record used only for the launch it was
taken on."""
import argparse
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _run("--steps", "1", "--warmup", "0", "--cpu-rows", "0")
    assert r.returncode != 0
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""


def _args(**kw):
    d = dict(gpus=1, steps=10, warmup=3, workload="large", rope="fused", adaln="token",
             pairing=None, kv_split=0, cpu_rows=8192, copy_calibration=False)
    d.update(kw)
    return argparse.Namespace(**d)


def test_traffic_record_only_for_its_own_launch():
    import bench
    from spatiotemporal_attention_vx_amd import configs
    path = os.path.join(ROOT, "profiles", "attention_large_traffic.json")
    with open(path) as f:
        rec = json.load(f)
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        current = hashlib.sha256(f.read()).hexdigest() == rec["source_sha256"]
    large, mixed = configs.get("large"), configs.get("mixed")
    got = bench.measured_traffic(large, _args(), 0)
    assert got == (rec["bytes_per_launch"] if current else None)
    # any other launch shape reports null, never the record's bytes
    assert bench.measured_traffic(mixed, _args(workload="mixed"), 0) is None
    assert bench.measured_traffic(large, _args(kv_split=37811), 0) is None
    assert bench.measured_traffic(large, _args(rope="separate"), 0) is None
    assert bench.measured_traffic(large, _args(), 2) is None


def test_traffic_record_is_consistent():
    """bytes_per_launch is the scaled sum of the two counters it records."""
    with open(os.path.join(ROOT, "profiles", "attention_large_traffic.json")) as f:
        rec = json.load(f)
    scaled = (rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024
    assert abs(scaled - rec["bytes_per_launch"]) <= 1e-4 * rec["bytes_per_launch"]
