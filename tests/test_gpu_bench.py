"""bench.py end to end on the GPU, a few steps: the JSON line's contract, and
the step of several library calls timed as replays of one captured HIP graph
(bench.py itself raises when a replay's outputs differ from the eager
step's)."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import announce

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", "--no-cpu-baseline",
           "--cold-reps", "0", "--no-onchip-ceiling", *args]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("workload,graph", [("detr", True), ("tsa", False), ("detr_encoder6", True),
                                            ("tsa_gridplan", False)])
def test_bench_line(workload, graph):
    announce(f"bench.py --workload {workload}")
    d = run_bench("--workload", workload)
    assert d["metric"] and d["unit"] == "samples/s" and d["n_gpus"] == 1 and d["steps"] == 3
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - d["samples_per_step"] / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    layers = 6 if workload == "detr_encoder6" else 1
    assert len(d["breakdown"]) == layers + (1 if workload == "detr" else 0)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and 0 < r["frac"] <= 1
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    if graph:
        assert d["launch"]["mode"].startswith("hip graph")
        assert d["launch"]["outputs_checked"] >= 1 and d["launch"]["replays"] == 3
        assert d["launch"]["eager"]["ms_per_step"] > 0
    else:
        assert d["launch"]["mode"].startswith("eager")
