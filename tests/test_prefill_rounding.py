"""Why bf16 prefill keeps its second (lo) P·V pass: a CPU emulation of the
kernel's rounding of the probabilities, checked against the parity gate.

The prefill kernel forms each probability p = 2^(s·scale·log2 e − m) in fp32,
sums the fp32 values into the softmax denominator, and feeds p to the bf16
matrix cores as hi = bf16(p) plus, for bf16, lo = bf16(p − hi).  Here every
other step is exact (fp64), so the only error besides the output rounding is
that of P:
  * hi + lo: p to about 16 significant bits -- inside the gate on every
    shape, with the same worst element as exact P;
  * hi alone: 8 bits -- the per-element bound fails (rows that see few keys
    put nearly all their weight on one or two rounded probabilities).
The shapes are those of tests/test_gpu_prefill.py (bf16, causal), drawn
from the same generator.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import ABS_TOL, RMS_TOL, ulp

SHAPES = [
    # (cache lens, new tokens, Hq, Hkv, D)
    ([1, 7, 300, 64], [1, 7, 300, 64], 8, 2, 128),
    ([130, 70], [130, 70], 4, 4, 128),
    ([96, 95, 97], [96, 50, 97], 6, 2, 64),
]


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def emulate(x, vq, mode):
    """Causal attention of every new token with P as the kernel rounds it."""
    s = x.spec
    q = vq.q.double().numpy()
    k = x.k.double().numpy()
    v = x.v.double().numpy()
    cq, ck = vq.cu_q.numpy(), x.cu_seqlens.numpy()
    out = np.zeros((vq.total_q, s.num_q_heads, s.head_dim_v))
    for b in range(s.batch):
        nq, lk = int(cq[b + 1] - cq[b]), int(ck[b + 1] - ck[b])
        for i in range(nq):
            L = lk - nq + i + 1
            if L <= 0:
                continue
            t = int(cq[b]) + i
            for h in range(s.num_q_heads):
                g = h // s.group
                sc = k[ck[b]:ck[b] + L, g] @ q[t, h] * s.scale
                p = np.exp(sc - sc.max()).astype(np.float32).astype(np.float64)  # fp32 probabilities
                hi = bf16(p)
                pr = hi + bf16(p - hi) if mode == "hi+lo" else hi
                out[t, h] = (pr @ v[ck[b]:ck[b] + L, g]) / p.sum()
    return out


def gate_ratios(out, ref):
    """(worst element / its bound, RMS / RMS budget) after rounding to bf16."""
    o = torch.from_numpy(out.astype(np.float32)).to(torch.bfloat16).double().numpy()
    err = np.abs(o - ref)
    bound = ABS_TOL + 0.5 * ulp(ref, torch.bfloat16)
    fmt = torch.from_numpy(ref).to(torch.bfloat16).double().numpy() - ref
    rms, rms_fmt = math.sqrt(float(np.mean(err ** 2))), math.sqrt(float(np.mean(fmt ** 2)))
    return float((err / bound).max()), rms / (RMS_TOL + rms_fmt)


@pytest.mark.parametrize("lens,q_lens,Hq,Hkv,D", SHAPES)
def test_bf16_prefill_needs_the_lo_pass(lens, q_lens, Hq, Hkv, D):
    spec = workloads.Spec("prefill", "gqa", len(lens), Hq, Hkv, D, D, tuple(lens), "bf16",
                          float(np.float32(1 / math.sqrt(D))), 11)
    x = workloads.make_inputs(spec)
    vq = workloads.make_varlen_query(x, q_lens, seed=11)
    qb = vq.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    ref, _ = oracle.gqa_varlen(qb, x.bits("k"), x.bits("v"), vq.cu_q.numpy(), x.cu_seqlens.numpy(), Hkv,
                               spec.scale, oracle.BF16, causal=True)
    both = gate_ratios(emulate(x, vq, "hi+lo"), ref)
    hi = gate_ratios(emulate(x, vq, "hi"), ref)
    assert both[0] < 0.85 and both[1] < 0.6, both    # hi + lo: inside the gate with margin
    assert hi[0] > both[0], (hi, both)               # hi alone is worse ...
    if D == 128:
        assert hi[0] > 1.0, hi                       # ... and breaks the per-element bound
