"""bench.py keeps its one-JSON-line contract: the keys, the roofline and CPU
baseline objects, and the refusal of a multi-GPU run (the library runs on one
GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_line_has_the_contract_keys():
    cmd = [sys.executable, BENCH, "--workload", "tiny_p128_r64_n4_gqa2_d64", "--steps", "2",
           "--warmup", "1", "--cpu-seconds", "1", "--no-mfma-peak"]
    print("case bench contract:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert out["unit"] == "TFLOP/s" and out["dtype"] == "bf16" and out["vs_baseline"] is None
    assert out["config"]["workload"] == "tiny_p128_r64_n4_gqa2_d64"
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2516.6
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert "traffic" in roof
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["unit"] == "TFLOP/s" and cpu["sample"]
    det = out["deterministic"]
    assert det["ms_per_step"] > 0 and det["bwd_workspace_gb"] > 0
    assert out["replicated"]["ms_per_step"] > 0
