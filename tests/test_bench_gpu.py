"""bench.py's one JSON line, run on the GPU for a few steps of the small 16-bit workload, the default
fp16 d256 causal workload and the e4m3 workload: the fields the line promises, and a roofline time that
cannot exceed the step time."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
          "vs_baseline", "dtype", "data", "config", "roofline")


def _line(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]  # exactly one JSON line
    return json.loads(lines[0])


@pytest.mark.gpu
@pytest.mark.parametrize("config,dtype,peak", [(2, "bf16", 2500.0), (4, "f16", 2500.0), (5, "fp8_e4m3", 5000.0)])
def test_bench_line_fields_and_roofline(config, dtype, peak):
    print(f"bench.py --config {config} --steps 3 --warmup 2", flush=True)
    d = _line("--config", str(config), "--steps", "3", "--warmup", "2", "--no-cpu-baseline")
    for k in FIELDS:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["dtype"] == dtype and "workload" in d["config"]
    assert 0 < d["value"] < peak
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["peak"] == peak and rf["unit"] == "TFLOP/s"
    assert 0 < rf["frac"] <= 1 and abs(rf["frac"] - rf["achieved"] / peak) < 1e-3
    # the dominant kernel's time per launch lies inside the step that contains it
    assert rf["kernel_avg_ms"] <= d["ms_per_step"] * 1.02
    assert rf["settled"]["median_ms"] > 0 and rf["cold_kernel_ms"] > 0
