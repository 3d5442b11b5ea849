"""bench.py's output contract on a GPU: one JSON line with the fields the
line is read by, run as its own process on the small workload (4,096 tokens,
8 heads x 128) so that it takes seconds."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_one_json_line_with_the_contract_fields(gpu_lib):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "small",
                        "--steps", "2", "--warmup", "1", "--cpu-rows", "8"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", float),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                     ("data", str), ("config", dict), ("roofline", dict),
                     ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), (key, d.get(key))
    assert "vs_baseline" in d
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["unit"] == "TFLOP/s" and d["dtype"] == "bf16"
    assert d["config"]["workload"].startswith("small")
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf and rf["traffic"] is None        # recorded for the large launch only
    assert "measured_ceiling" not in rf
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert isinstance(cb["unit"], str) and "8 seeded query rows" in cb["sample"]
    k = d["kernels"]
    assert k["attn_ms"] > 0 and k["adaln_ms"] > 0 and k["rope_ms"] > 0
