"""bench.py end to end on the GPU, a few steps of small workloads: the one
JSON line carries every field of the reporting contract, with values that
are consistent with each other."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}


def bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("args", [("--workload", "2"), ("--workload", "1", "--window", "64")])
def test_bench_line(args):
    res = bench(*args, "--steps", "5", "--warmup", "3")
    assert KEYS <= set(res)
    assert res["n_gpus"] == 1 and res["steps"] == 5 and res["warmup"] == 3
    assert res["unit"] == "tokens/s" and res["value"] > 0 and res["ms_per_step"] > 0
    cfg = res["config"]
    assert cfg["workload"] and "model" not in cfg
    roof = res["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = res["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["cpu_model"] and cpu["cpus_online"] >= cpu["cores"]
    whole = res["whole_call"]
    assert whole["flushed_ms_median"] > 0
