"""CPU checks of the benchmark harness: it measures one GPU only and says so
for any other count, and its oracle baseline leg reports a rate in the
metric's unit with the thread count it used."""
import json
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert p.returncode == 2
    rec = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in rec["error"] and rec["n_gpus_requested"] == int(n)


def test_oracle_baseline_leg_reports_rate_and_threads():
    sys.path.insert(0, ROOT)
    import bench
    spec = workloads.with_shape(workloads.WORKLOADS[1], batch=3, lens=(40, 7, 100))
    x = workloads.make_inputs(spec)
    rec = bench.oracle_rate(x, spec, 0.05, 1)
    assert rec["unit"] == "GB/s" and rec["value"] > 0 and rec["cores"] == 1
    assert rec["kind"] == "oracle" and "sample" in rec
