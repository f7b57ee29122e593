"""bench.py's output contract: one JSON line with the metric, the whole-job value, the step
timing, and the roofline and CPU-baseline objects (a short run: few steps, no detail)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*extra):
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "3",
                          "--no-detail", *extra], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, out.stdout
    return json.loads(lines[0])


def test_bench_json_contract():
    r = _bench()
    for key, kind in (("metric", str), ("value", (int, float)), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", (int, float)), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(r[key], kind), key
    assert r["n_gpus"] == 1 and r["steps"] == 3 and r["warmup"] == 3 and r["value"] > 0
    assert r["vs_baseline"] is None and r["config"]["workload"] == "1mp_dense"
    roof = r["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    # the MFMA probe's rates: repeating operands, random bf16 operands (lower: a lower clock), i8
    peak = roof["measured_mfma_peak"]
    assert 0 < peak["bf16_random_operands_tflops"] <= peak["bf16_tflops"] * 1.02 and peak["i8_tops"] > 0
    assert roof["frac_of_measured_peak"] <= roof["frac_of_random_operand_peak"] * 1.02
    cpu = r["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]


def test_bench_refuses_more_than_one_gpu():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert out.returncode != 0 and "one GPU" in out.stderr
