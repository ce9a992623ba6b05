"""GPU parity of the prefill kernel (zl_attn_prefill_gqa, through the C ABI)
against the fp64 oracle on identical seeded inputs: whole prompts, chunks of
prompts, mixed batches, no mask, more new tokens than cache rows, empty
sequences, G from 1 to 8, both head dims and both 16-bit types; a long
prompt and a long chunk on every row.  Outputs are pre-filled with NaN /
+inf and surrounded by canaries (tests/guard.py)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.guard import CallBuffers
from tests.parity import gate

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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


def make(lens, q_lens, Hq, Hkv, D, dt, seed=11):
    spec = workloads.Spec("prefill", "gqa", len(lens), Hq, Hkv, D, D, tuple(lens),
                          "f16" if dt == torch.float16 else "bf16", float(np.float32(1 / math.sqrt(D))), seed)
    x = workloads.make_inputs(spec)
    return x, workloads.make_varlen_query(x, q_lens, seed=seed)


def run(x, vq, causal=True, where=""):
    bufs = CallBuffers(vq.total_q, x.spec.num_q_heads, x.spec.head_dim_v, x.spec.torch_dtype, DEV)
    out, lse = zl().zl_attn_prefill_gqa(vq.q.to(DEV), x.k.to(DEV), x.v.to(DEV), vq.cu_q.to(DEV),
                                        x.cu_seqlens.to(DEV), x.max_seqlen, x.spec.scale, causal=causal,
                                        **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check(where)
    return out, lse


def oracle_rows(x, vq, causal=True, rows=None):
    qb = vq.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    dt = oracle.F16 if x.spec.torch_dtype == torch.float16 else oracle.BF16
    return oracle.gqa_varlen(qb, x.bits("k"), x.bits("v"), vq.cu_q.numpy(), x.cu_seqlens.numpy(),
                             x.spec.num_kv_heads, x.spec.scale, dt, causal=causal, rows=rows)


CASES = [
    # (cache lens, new tokens, Hq, Hkv, D, dtype)
    ([1, 7, 300, 64], [1, 7, 300, 64], 8, 2, 128, torch.bfloat16),     # whole prompts
    ([500, 1000], [128, 37], 16, 4, 128, torch.float16),               # chunks of prompts
    ([200, 33], [200, 33], 8, 1, 64, torch.float16),                   # G = 8
    ([130, 70], [130, 70], 4, 4, 128, torch.bfloat16),                 # G = 1
    ([96, 95, 97], [96, 50, 97], 6, 2, 64, torch.bfloat16),            # G = 3
    ([3, 40], [9, 40], 4, 2, 128, torch.float16),                      # more new tokens than rows
    ([0, 50, 60, 0], [0, 50, 0, 3], 8, 2, 128, torch.float16),         # empty sequences
    ([(i * 37) % 90 + 1 for i in range(70)], [(i * 11) % 40 for i in range(70)], 8, 2, 128, torch.bfloat16),
]


@pytest.mark.parametrize("lens,q_lens,Hq,Hkv,D,dt", CASES)
def test_prefill_parity(lens, q_lens, Hq, Hkv, D, dt):
    x, vq = make(lens, q_lens, Hq, Hkv, D, dt)
    where = f"prefill {lens[:5]} q {q_lens[:5]} {Hq}/{Hkv} D{D} {dt}"
    print(where, flush=True)
    out, lse = run(x, vq, where=where)
    ro, rl = oracle_rows(x, vq)
    gate(out, ro, dt, lse, rl, where=where)


def test_prefill_without_mask():
    x, vq = make([300, 41], [100, 41], 8, 2, 128, torch.float16)
    out, lse = run(x, vq, causal=False)
    ro, rl = oracle_rows(x, vq, causal=False)
    gate(out, ro, torch.float16, lse, rl, where="prefill, no mask")


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_prefill_negative_and_zero_scale(scale):
    """A negative softmax scale (the kernel moves its sign onto the query
    operands) and a zero scale (uniform weights over the visible keys)."""
    x, vq = make([300, 41], [100, 41], 8, 2, 128, torch.bfloat16)
    x.spec = dataclasses.replace(x.spec, scale=float(np.float32(scale)))
    out, lse = run(x, vq)
    ro, rl = oracle_rows(x, vq)
    gate(out, ro, torch.bfloat16, lse, rl, where=f"prefill, scale {scale}")


@pytest.mark.skip(reason="the GPU faulted in this test under a start-up variant of the decode and merge "
                         "kernels (since taken out) and no cause was found; off the GPU until one is shown. "
                         "Both paths keep their own oracle parity tests.")
def test_prefill_agrees_with_the_several_tokens_path():
    """The two kernels for several new tokens give the same attention (within
    rounding) on the same inputs."""
    x, vq = make([700, 260], [300, 260], 32, 8, 128, torch.bfloat16)
    out, _ = run(x, vq)
    ref = zl().zl_attn_varlen_gqa(vq.q.to(DEV), x.k.to(DEV), x.v.to(DEV), vq.cu_q.to(DEV), x.cu_seqlens.to(DEV),
                                  x.max_seqlen, x.spec.scale)
    torch.cuda.synchronize()
    assert (out.float() - ref.float()).abs().max().item() < 8e-3


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_long_prompt_every_row(dt):
    """One 4096-token prompt and one 1024-token chunk after 3072 cached tokens,
    32 query / 8 key-value heads, D 128: every (token, head) row against the
    oracle."""
    x, vq = make([4096, 4096], [4096, 1024], 32, 8, 128, dt, seed=5)
    where = f"long prompt {dt}"
    print(where, flush=True)
    out, lse = run(x, vq, where=where)
    ro, rl = oracle_rows(x, vq)
    gate(out, ro, dt, lse, rl, where=where)


# ------------------------------------------------------------ paged caches
def run_paged(x, vq, px, causal=True, where=""):
    bufs = CallBuffers(vq.total_q, x.spec.num_q_heads, x.spec.head_dim_v, x.spec.torch_dtype, DEV)
    out, lse = zl().zl_attn_prefill_gqa_paged(vq.q.to(DEV), px.k_pages.to(DEV), px.v_pages.to(DEV),
                                              px.block_table.to(DEV), vq.cu_q.to(DEV), x.cu_seqlens.to(DEV),
                                              x.max_seqlen, x.spec.scale, causal=causal, **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check(where)
    return out, lse


PAGED_CASES = [
    # (cache lens, new tokens, Hq, Hkv, D, dtype, page size)
    ([1, 7, 300, 64], [1, 7, 300, 64], 8, 2, 128, torch.bfloat16, 16),    # whole prompts, 16-token pages
    ([500, 1000], [128, 37], 16, 4, 128, torch.float16, 64),              # chunks after a cached prefix
    ([200, 33], [200, 33], 8, 1, 64, torch.float16, 32),
    ([130, 70], [130, 70], 4, 4, 128, torch.bfloat16, 256),
    ([96, 95, 97], [96, 50, 97], 6, 2, 64, torch.bfloat16, 16),
    ([3, 40], [9, 40], 4, 2, 128, torch.float16, 16),                     # more new tokens than rows
    ([0, 50, 60, 0], [0, 50, 0, 3], 8, 2, 128, torch.float16, 128),       # empty sequences
    ([(i * 37) % 90 + 1 for i in range(70)], [(i * 11) % 40 for i in range(70)], 8, 2, 128, torch.bfloat16, 16),
]


@pytest.mark.parametrize("lens,q_lens,Hq,Hkv,D,dt,ps", PAGED_CASES)
def test_paged_prefill(lens, q_lens, Hq, Hkv, D, dt, ps):
    """Against the oracle on every row, and bitwise equal to packed prefill on
    the same rows (the pages change where rows live, not the arithmetic)."""
    x, vq = make(lens, q_lens, Hq, Hkv, D, dt)
    px = workloads.make_paged(x, ps, seed=ps + len(lens))
    where = f"paged prefill {lens[:5]} q {q_lens[:5]} {Hq}/{Hkv} D{D} {dt} ps{ps}"
    print(where, flush=True)
    out, lse = run_paged(x, vq, px, where=where)
    ro, rl = oracle_rows(x, vq)
    gate(out, ro, dt, lse, rl, where=where)
    po, pl = run(x, vq, where=where + " (packed)")
    assert torch.equal(out, po) and torch.equal(lse, pl), where


def test_paged_prefill_without_mask():
    x, vq = make([300, 41], [100, 41], 8, 2, 128, torch.float16)
    px = workloads.make_paged(x, 16, seed=4)
    out, lse = run_paged(x, vq, px, causal=False, where="paged prefill, no mask")
    ro, rl = oracle_rows(x, vq, causal=False)
    gate(out, ro, torch.float16, lse, rl, where="paged prefill, no mask")


@pytest.mark.parametrize("ps", [16, 256])
def test_paged_long_prompt_every_row(ps):
    """The long-prompt case over a shuffled page pool: a 4096-token prompt and a
    1024-token chunk after 3072 cached tokens, every row against the oracle."""
    x, vq = make([4096, 4096], [4096, 1024], 32, 8, 128, torch.bfloat16, seed=5)
    px = workloads.make_paged(x, ps, seed=9)
    where = f"paged long prompt ps{ps}"
    print(where, flush=True)
    out, lse = run_paged(x, vq, px, where=where)
    ro, rl = oracle_rows(x, vq)
    gate(out, ro, torch.bfloat16, lse, rl, where=where)
    po, _ = run(x, vq)
    assert torch.equal(out, po)


MANY = [
    # (query heads, key/value heads, head dim, dtype, causal, page size)
    (32, 8, 128, torch.bfloat16, True, 0),
    (32, 8, 128, torch.bfloat16, True, 16),
    (8, 8, 64, torch.float16, True, 0),       # G = 1, D = 64
    (16, 2, 64, torch.bfloat16, False, 64),   # no mask, D = 64, 64-token pages
    (24, 3, 128, torch.float16, True, 0),     # G = 8
]


@pytest.mark.parametrize("Hq,Hkv,D,dt,causal,ps", MANY)
def test_many_sequences_many_rounds(Hq, Hkv, D, dt, causal, ps):
    """80 ragged sequences: hundreds to thousands of blocks, so the 512
    resident workgroups take several each, over the batch's second chunk of
    64 sequences too; some sequences have more new tokens than cache rows
    (their first blocks see no key) and some none.  Every row against the
    oracle, packed or over pages."""
    lens = [(i * 53) % 400 + 1 for i in range(80)]
    q_lens = [0 if i % 17 == 5 else min(lens[i] + (i % 3) * 40, (i * 29) % 300 + 1) for i in range(80)]
    x, vq = make(lens, q_lens, Hq, Hkv, D, dt, seed=23)
    where = f"80 sequences, {Hq}/{Hkv} heads, D {D}, causal {causal}, pages {ps}"
    print(where, flush=True)
    if ps:
        out, lse = run_paged(x, vq, workloads.make_paged(x, ps), causal=causal, where=where)
    else:
        out, lse = run(x, vq, causal=causal, where=where)
    ro, rl = oracle_rows(x, vq, causal=causal)
    gate(out, ro, dt, lse, rl, where=where)


def test_repeated_calls_are_bitwise_identical():
    """The persistent schedule is fixed by the shapes alone: five calls over
    the 80-sequence batch give the same bits (and the same lse)."""
    lens = [(i * 53) % 400 + 1 for i in range(80)]
    q_lens = [min(lens[i] + (i % 3) * 40, (i * 29) % 300 + 1) for i in range(80)]
    x, vq = make(lens, q_lens, 32, 8, 128, torch.float16, seed=29)
    first = None
    for k in range(5):
        out, lse = run(x, vq, where=f"repeat {k}")
        got = (out.view(torch.int16).cpu(), lse.cpu())
        if first is None:
            first = got
        else:
            assert torch.equal(got[0], first[0]) and torch.equal(got[1].view(torch.int32), first[1].view(torch.int32)), k
