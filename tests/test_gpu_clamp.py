"""Cache lengths are clamped inside the kernels: sequence b attends over its
first clamp(cu[b+1] - cu[b], 0, max_seqlen_k) rows, from cache row cu[b].
Each case calls the library with an unchecked cu (starting above 0,
decreasing, lengths above max_seqlen_k) on a packed cache that holds every
row cu names, and compares every output row with the oracle run on the
clamped rows gathered into a valid batch.  A read past the clamp would pick
up the cache's further random rows and fail the gate.

Paged caches are covered on the CPU (tests/test_split_model.py: block-table
reads stay below ceil(max_seqlen_k / page_size) whatever cu holds).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.guard import CallBuffers
from tests.parity import gate
from tests.test_gpu_parity import DEV, odt, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_amd as zl
    zl.library()
    yield


def zl():
    import mla_attention_amd
    return mla_attention_amd


def walk(start, steps):
    """cu values from `start` by the given steps, floored at 0 (decreasing
    stretches and lengths above any clamp included)."""
    cu = [start]
    for d in steps:
        cu.append(max(0, cu[-1] + d))
    return cu


def spec(kind, batch, Hq, Hkv, D, dt, seed):
    d = "f16" if dt == torch.float16 else "bf16"
    if kind == "mla":
        return workloads.Spec("clamp-mla", "mla", batch, Hq, 1, 576, 512, (1,) * batch, d,
                              float(np.float32(1 / math.sqrt(192))), seed)
    return workloads.Spec("clamp-gqa", "gqa", batch, Hq, Hkv, D, D, (1,) * batch, d,
                          float(np.float32(1 / math.sqrt(D))), seed)


def ws_bytes(s, M):
    if s.kind == "mla":
        return zl().zl_decode_attn_mla_workspace_size(s.batch, s.num_q_heads, 512, 64, M, s.torch_dtype)
    return zl().zl_decode_attn_workspace_size(s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim_k, M,
                                              s.torch_dtype)


def decode_call(rc, where=""):
    """One decode call on the raw cu."""
    x = rc.clamped
    s = x.spec
    bufs = CallBuffers(s.batch, s.num_q_heads, s.head_dim_v, s.torch_dtype, DEV, ws_bytes(s, rc.max_seqlen))
    q, cu, M = x.q.to(DEV), rc.cu_raw.to(DEV), rc.max_seqlen
    if s.kind == "mla":
        out, lse = zl().zl_decode_attn_mla(q, rc.latent.to(DEV), cu, M, s.scale, **bufs.kwargs())
    else:
        out, lse = zl().zl_decode_attn_gqa(q, rc.k.to(DEV), rc.v.to(DEV), cu, M, s.scale, **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check(where)
    return out, lse


DECODE = [
    # (kind, cu, max_seqlen_k, Hq, Hkv, D, dtype)
    ("gqa", [5, 705, 745, 300, 1200, 1200, 1233], 600, 8, 2, 128, torch.float16),
    ("gqa", walk(100, [((i * 97) % 420) - 60 for i in range(80)]), 256, 4, 4, 64, torch.bfloat16),
    ("gqa", [0, 300, 310, 200, 700], 128, 32, 1, 64, torch.float16),            # G = 32: two head blocks
    ("gqa", [7, 7, 3, 2000], 1000, 8, 1, 128, torch.bfloat16),                  # empty, negative, long
    ("mla", [3, 900, 950, 400, 1500, 1530], 700, 16, 1, 576, torch.bfloat16),
    ("mla", walk(50, [((i * 131) % 300) - 40 for i in range(70)]), 200, 16, 1, 576, torch.float16),
]
DECODE_IDS = [f"{c[0]}-B{len(c[1]) - 1}-M{c[2]}-H{c[3]}" for c in DECODE]


@pytest.mark.parametrize("kind,cu,M,Hq,Hkv,D,dt", DECODE, ids=DECODE_IDS)
def test_decode_clamps_lengths(kind, cu, M, Hq, Hkv, D, dt):
    rc = workloads.make_raw_cache(spec(kind, len(cu) - 1, Hq, Hkv, D, dt, 31), cu, M, seed=31)
    where = f"clamp decode {kind} cu[:8]={cu[:8]} M={M}"
    print(where, flush=True)
    out, lse = decode_call(rc, where=where)
    ro, rl = run_oracle(rc.clamped)
    gate(out, ro, dt, lse, rl, where=where)


VARLEN = [
    # (kind, cu_k, max_seqlen_k, new tokens, Hq, Hkv, D, dtype)
    ("gqa", [5, 705, 745, 300, 1200, 1200, 1233], 600, [3, 1, 0, 5, 0, 2], 8, 2, 128, torch.float16),
    ("gqa", [0, 300, 310, 200, 700], 128, [2, 7, 0, 1], 32, 1, 64, torch.bfloat16),
    ("mla", [3, 900, 950, 400, 1500, 1530], 700, [2, 1, 0, 4, 3], 16, 1, 576, torch.bfloat16),
]


def varlen_call(rc, vq, causal, where=""):
    x = rc.clamped
    s = x.spec
    bufs = CallBuffers(vq.total_q, s.num_q_heads, s.head_dim_v, s.torch_dtype, DEV, ws_bytes(s, rc.max_seqlen))
    q, cq, ck, M = vq.q.to(DEV), vq.cu_q.to(DEV), rc.cu_raw.to(DEV), rc.max_seqlen
    kw = dict(causal=causal, **bufs.kwargs())
    if s.kind == "mla":
        out, lse = zl().zl_attn_varlen_mla(q, rc.latent.to(DEV), cq, ck, M, s.scale, **kw)
    else:
        out, lse = zl().zl_attn_varlen_gqa(q, rc.k.to(DEV), rc.v.to(DEV), cq, ck, M, s.scale, **kw)
    torch.cuda.synchronize()
    bufs.check(where)
    return out, lse


def varlen_oracle(x, vq, causal):
    s = x.spec
    qb = vq.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    cq, ck = vq.cu_q.numpy(), x.cu_seqlens.numpy()
    if s.kind == "mla":
        return oracle.mla_varlen(qb, x.bits("latent"), cq, ck, s.scale, odt(s), causal=causal)
    return oracle.gqa_varlen(qb, x.bits("k"), x.bits("v"), cq, ck, s.num_kv_heads, s.scale, odt(s), causal=causal)


@pytest.mark.parametrize("kind,cu,M,q_lens,Hq,Hkv,D,dt", VARLEN)
def test_several_new_tokens_clamp_lengths(kind, cu, M, q_lens, Hq, Hkv, D, dt):
    """The causal mask counts positions in the clamped cache: new token i of
    sequence b sits at L_b - nq + i."""
    rc = workloads.make_raw_cache(spec(kind, len(cu) - 1, Hq, Hkv, D, dt, 33), cu, M, seed=33)
    vq = workloads.make_varlen_query(rc.clamped, q_lens, seed=33)
    where = f"clamp varlen {kind} cu={cu} M={M} q={q_lens}"
    print(where, flush=True)
    out, lse = varlen_call(rc, vq, True, where=where)
    ro, rl = varlen_oracle(rc.clamped, vq, True)
    gate(out, ro, dt, lse, rl, where=where)


def test_prefill_clamps_lengths():
    cu, M = [5, 705, 745, 300, 1200, 1200, 1233], 600
    rc = workloads.make_raw_cache(spec("gqa", 6, 8, 2, 128, torch.bfloat16, 34), cu, M, seed=34)
    vq = workloads.make_varlen_query(rc.clamped, [600, 40, 0, 300, 0, 33], seed=34)
    s = rc.clamped.spec
    bufs = CallBuffers(vq.total_q, s.num_q_heads, s.head_dim_v, s.torch_dtype, DEV)
    print("clamp prefill", flush=True)
    out, lse = zl().zl_attn_prefill_gqa(vq.q.to(DEV), rc.k.to(DEV), rc.v.to(DEV), vq.cu_q.to(DEV),
                                        rc.cu_raw.to(DEV), M, s.scale, causal=True, **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check("clamp prefill")
    ro, rl = varlen_oracle(rc.clamped, vq, True)
    gate(out, ro, s.torch_dtype, lse, rl, where="clamp prefill")
