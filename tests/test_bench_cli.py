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


def test_prefill_oracle_baseline_counts_the_sample_flops():
    """The sample's flops are the causal keys of its rows: with one prompt of
    n tokens and every row sampled, they equal the whole step's."""
    sys.path.insert(0, ROOT)
    import bench
    n = 24
    spec = workloads.with_shape(workloads.WORKLOADS[1], batch=1, lens=(n,))
    x = workloads.make_inputs(spec)
    vq = workloads.make_varlen_query(x, [n], seed=1)
    step_flops = 4.0 * spec.num_q_heads * spec.head_dim_k * n * (n + 1) / 2
    rec = bench.cpu_baseline_prefill(x, vq, spec, step_flops, 0.02)
    assert rec["unit"] == "TFLOP/s" and rec["value"] > 0 and rec["kind"] == "oracle"
    # n tokens by 8 heads: every row of the prompt (24 tokens, 8 heads)
    assert f"{n * spec.num_q_heads} (new token, head) rows" in rec["sample"]
    assert f"{step_flops:.4g} useful flops" in rec["sample"]


@pytest.mark.parametrize("mode", ["quantize", "dequantize", "reduce"])
def test_codec_oracle_baseline_reports_bytes_per_second(mode):
    sys.path.insert(0, ROOT)
    import bench
    import torch
    base = torch.randn(4096, generator=torch.Generator().manual_seed(0)).to(torch.float16)
    rec = bench.cpu_baseline_codec(mode, base, 512, 3.0, 0.01)
    assert rec["unit"] == "GB/s" and rec["value"] > 0 and rec["cores"] == 1 and rec["kind"] == "oracle"
