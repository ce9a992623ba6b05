"""GPU parity for several new query tokens per sequence (chunked prefill,
draft tokens): the HIP kernels through the C ABI against the fp64 oracle on
identical seeded inputs.

Every case compares every (token, head) row, the full-size draft-token
batches included.  One new token per sequence must give the decode path's
bits exactly.  Outputs are pre-filled with NaN / +inf and surrounded by
canaries (tests/guard.py).
"""
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


def odt(dtype):
    return oracle.F16 if dtype == torch.float16 else oracle.BF16


def spec_gqa(lens, Hq, Hkv, D, dt, seed=7):
    return workloads.Spec("varlen", "gqa", len(lens), Hq, Hkv, D, D, tuple(lens),
                          "f16" if dt == torch.float16 else "bf16", float(np.float32(1 / math.sqrt(D))), seed)


def spec_mla(lens, H, dt, seed=9):
    return workloads.Spec("varlen-mla", "mla", len(lens), H, 1, 576, 512, tuple(lens),
                          "f16" if dt == torch.float16 else "bf16", float(np.float32(1 / math.sqrt(192))), seed)


def buffers(x, vq, num_workers=0):
    """Guarded out / lse / workspace for one call."""
    s = x.spec
    if s.kind == "mla":
        ws = zl().zl_decode_attn_mla_workspace_size(s.batch, s.num_q_heads, 512, 64, x.max_seqlen, s.torch_dtype,
                                                    num_workers)
    else:
        ws = zl().zl_decode_attn_workspace_size(s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim_k, x.max_seqlen,
                                                s.torch_dtype, num_workers)
    return CallBuffers(vq.total_q, s.num_q_heads, s.head_dim_v, s.torch_dtype, DEV, ws)


def run_gpu(x, vq, causal=True, num_workers=0, where=""):
    s = x.spec
    q = vq.q.to(DEV)
    cq, ck = vq.cu_q.to(DEV), x.cu_seqlens.to(DEV)
    bufs = buffers(x, vq, num_workers)
    if s.kind == "mla":
        out, lse = zl().zl_attn_varlen_mla(q, x.latent.to(DEV), cq, ck, x.max_seqlen, s.scale, causal=causal,
                                           num_workers=num_workers, **bufs.kwargs())
    else:
        out, lse = zl().zl_attn_varlen_gqa(q, x.k.to(DEV), x.v.to(DEV), cq, ck, x.max_seqlen, s.scale,
                                           causal=causal, num_workers=num_workers, **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check(where)
    return out, lse


def run_oracle(x, vq, causal=True, rows=None):
    s = x.spec
    qb = vq.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    cq, ck = vq.cu_q.numpy(), x.cu_seqlens.numpy()
    if s.kind == "mla":
        return oracle.mla_varlen(qb, x.bits("latent"), cq, ck, s.scale, odt(s.torch_dtype), causal=causal,
                                 rows=rows)
    return oracle.gqa_varlen(qb, x.bits("k"), x.bits("v"), cq, ck, s.num_kv_heads, s.scale, odt(s.torch_dtype),
                             causal=causal, rows=rows)


def check(x, vq, where, causal=True, **kw):
    print(where, flush=True)
    out, lse = run_gpu(x, vq, causal, where=where, **kw)
    ro, rl = run_oracle(x, vq, causal)
    return gate(out, ro, x.spec.torch_dtype, lse, rl, where=where)


GQA_CASES = [
    # (cache lens, new tokens per sequence, Hq, Hkv, D, dtype)
    ([17, 64, 100, 128], [1, 2, 3, 4], 8, 2, 64, torch.float16),
    ([100, 1, 300, 64, 33], [100, 1, 37, 0, 33], 8, 2, 128, torch.bfloat16),   # prefill, decode, chunk, none
    ([200, 150], [4, 4], 32, 8, 128, torch.float16),                          # G*q = 16: one row block
    ([129, 70], [2, 3], 32, 1, 64, torch.float16),                            # G = 32: blocks of 16 rows
    ([96, 95, 97], [5, 1, 6], 6, 2, 128, torch.bfloat16),                    # G = 3: blocks across tokens
    ([3, 40], [5, 2], 4, 4, 64, torch.float16),                               # more new tokens than rows
    ([0, 50, 0], [2, 3, 0], 8, 2, 128, torch.float16),                        # empty caches
    ([(i * 37) % 90 for i in range(80)], [(i * 7) % 4 for i in range(80)], 8, 2, 128, torch.bfloat16),
]


@pytest.mark.parametrize("lens,q_lens,Hq,Hkv,D,dt", GQA_CASES)
def test_gqa_varlen(lens, q_lens, Hq, Hkv, D, dt):
    x = workloads.make_inputs(spec_gqa(lens, Hq, Hkv, D, dt))
    vq = workloads.make_varlen_query(x, q_lens, seed=len(lens))
    check(x, vq, f"gqa varlen {lens[:6]} q {q_lens[:6]} {Hq}/{Hkv} D{D} {dt}")


def test_gqa_varlen_without_mask():
    x = workloads.make_inputs(spec_gqa([40, 300, 7], 8, 2, 128, torch.float16))
    vq = workloads.make_varlen_query(x, [3, 20, 9], seed=3)
    check(x, vq, "gqa varlen, no mask", causal=False)


MLA_CASES = [
    ([40, 300, 1], [2, 1, 1], 16, torch.bfloat16),
    ([257, 33], [2, 2], 8, torch.float16),       # H*q = 16: one row block
    ([70, 150], [3, 1], 32, torch.bfloat16),
    ([5, 64], [9, 64], 16, torch.bfloat16),      # more new tokens than rows; a whole prompt
    ([(i * 53) % 90 for i in range(70)], [(i * 5) % 3 for i in range(70)], 16, torch.bfloat16),
    # MLA tiles serve blocks of 32 query rows (two MFMA column blocks):
    ([300, 45], [3, 5], 16, torch.float16),      # 48 and 80 rows: a half-full last block
    ([130], [4], 8, torch.bfloat16),             # 4 tokens (4 causal limits) in one block
    ([90, 200], [2, 2], 128, torch.float16),     # 8 blocks per sequence
    ([61, 0, 33], [1, 2, 1], 16, torch.float16), # an empty cache with new tokens
]


@pytest.mark.parametrize("lens,q_lens,H,dt", MLA_CASES)
def test_mla_varlen(lens, q_lens, H, dt):
    x = workloads.make_inputs(spec_mla(lens, H, dt))
    vq = workloads.make_varlen_query(x, q_lens, seed=len(lens))
    check(x, vq, f"mla varlen {lens[:6]} q {q_lens[:6]} H{H} {dt}")


def test_mla_varlen_without_mask():
    x = workloads.make_inputs(spec_mla([40, 300, 7], 16, torch.bfloat16))
    vq = workloads.make_varlen_query(x, [3, 20, 9], seed=4)
    check(x, vq, "mla varlen, no mask", causal=False)


@pytest.mark.parametrize("workers", [8, 64, 256, 2048])
def test_any_worker_count_gives_the_same_attention(workers):
    x = workloads.make_inputs(workloads.with_shape(workloads.WORKLOADS[2], batch=5, lens=("uniform", 1, 2000)),
                              seed=23)
    vq = workloads.make_varlen_query(x, [1, 4, 16, 2, 7], seed=5)
    check(x, vq, f"gqa varlen workers={workers}", num_workers=workers)
    xm = workloads.make_inputs(workloads.with_shape(workloads.WORKLOADS[5], batch=3, lens=("uniform", 1, 1500)),
                               seed=24)
    vqm = workloads.make_varlen_query(xm, [2, 1, 3], seed=6)
    check(xm, vqm, f"mla varlen workers={workers}", num_workers=workers)


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_one_new_token_gives_the_decode_bits(cfg):
    """With one new token per sequence the virtual sequences are the decode
    batch itself, so the arithmetic, and the bits, are those of decode."""
    x = workloads.make_inputs(workloads.WORKLOADS[cfg])
    vq = workloads.VarlenQuery(np.ones(x.spec.batch, dtype=np.int64),
                               workloads.cu_from_lens([1] * x.spec.batch), x.q.clone())
    out, lse = run_gpu(x, vq)
    cu = x.cu_seqlens.to(DEV)
    if x.spec.kind == "mla":
        ro, rl = zl().zl_decode_attn_mla(x.q.to(DEV), x.latent.to(DEV), cu, x.max_seqlen, x.spec.scale,
                                         return_lse=True)
    else:
        ro, rl = zl().zl_decode_attn_gqa(x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), cu, x.max_seqlen, x.spec.scale,
                                         return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ro) and torch.equal(lse, rl)


@pytest.mark.parametrize("cfg,q_len", [(2, 4), (3, 2), (4, 4), (5, 2)])
def test_full_size_draft_tokens_every_row(cfg, q_len):
    """Full-size batches with q_len new tokens per sequence (draft-token
    verification): every (token, head) row against the oracle."""
    spec = workloads.WORKLOADS[cfg]
    where = f"{spec.name}, {q_len} new tokens per sequence"
    x = workloads.make_inputs(spec)
    vq = workloads.make_varlen_query(x, [q_len] * spec.batch, seed=cfg)
    check(x, vq, where)


def run_gpu_paged(x, vq, px, causal=True, num_workers=0, where=""):
    s = x.spec
    q = vq.q.to(DEV)
    cq, ck, bt = vq.cu_q.to(DEV), x.cu_seqlens.to(DEV), px.block_table.to(DEV)
    bufs = buffers(x, vq, num_workers)
    if s.kind == "mla":
        out, lse = zl().zl_attn_varlen_mla_paged(q, px.kv_pages.to(DEV), bt, cq, ck, x.max_seqlen, s.scale,
                                                 causal=causal, num_workers=num_workers, **bufs.kwargs())
    else:
        out, lse = zl().zl_attn_varlen_gqa_paged(q, px.k_pages.to(DEV), px.v_pages.to(DEV), bt, cq, ck,
                                                 x.max_seqlen, s.scale, causal=causal, num_workers=num_workers,
                                                 **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check(where)
    return out, lse


def check_paged(x, vq, page_size, where, causal=True, num_workers=0):
    """Paged caches hold the packed caches' rows (the paged layout's
    definition, checked here on the pools themselves), so the oracle on the
    packed rows is the reference; the packed call, with the same split, must
    give the same bits."""
    print(where, flush=True)
    px = workloads.make_paged(x, page_size, seed=len(x.lens))
    cu = x.cu_seqlens.numpy()
    if x.spec.kind == "mla":
        assert np.array_equal(oracle.gather_paged(px.kv_pages.view(torch.int16).numpy(), px.block_table.numpy(),
                                                  cu, page_size), x.latent.view(torch.int16).numpy())
    else:
        assert np.array_equal(oracle.gather_paged(px.k_pages.view(torch.int16).numpy(), px.block_table.numpy(),
                                                  cu, page_size), x.k.view(torch.int16).numpy())
    out, lse = run_gpu_paged(x, vq, px, causal, num_workers, where=where)
    ro, rl = run_oracle(x, vq, causal)
    gate(out, ro, x.spec.torch_dtype, lse, rl, where=where)
    po, pl = run_gpu(x, vq, causal, num_workers)
    assert torch.equal(out, po) and torch.equal(lse, pl), where


PAGED_GQA_CASES = [
    # (cache lens, new tokens per sequence, Hq, Hkv, D, dtype, page size)
    ([17, 64, 100, 128], [1, 2, 3, 4], 8, 2, 64, torch.float16, 16),
    ([100, 1, 300, 64, 33], [100, 1, 37, 0, 33], 8, 2, 128, torch.bfloat16, 16),
    ([200, 150], [4, 4], 32, 8, 128, torch.float16, 64),
    ([96, 95, 97], [5, 1, 6], 6, 2, 128, torch.bfloat16, 32),
    ([0, 50, 0], [2, 3, 0], 8, 2, 128, torch.float16, 16),
    ([700, 260], [9, 3], 32, 8, 128, torch.bfloat16, 256),
    ([(i * 37) % 90 for i in range(80)], [(i * 7) % 4 for i in range(80)], 8, 2, 128, torch.bfloat16, 16),
]


@pytest.mark.parametrize("lens,q_lens,Hq,Hkv,D,dt,page", PAGED_GQA_CASES)
def test_gqa_varlen_paged(lens, q_lens, Hq, Hkv, D, dt, page):
    x = workloads.make_inputs(spec_gqa(lens, Hq, Hkv, D, dt))
    vq = workloads.make_varlen_query(x, q_lens, seed=len(lens))
    check_paged(x, vq, page, f"gqa varlen paged {lens[:6]} q {q_lens[:6]} {Hq}/{Hkv} D{D} {dt} page {page}")


PAGED_MLA_CASES = [
    ([40, 300, 1], [2, 1, 1], 16, torch.bfloat16, 16),
    ([300, 45], [3, 5], 16, torch.float16, 64),
    ([5, 64], [9, 64], 16, torch.bfloat16, 16),
    ([61, 0, 33], [1, 2, 1], 16, torch.float16, 32),
    ([90, 200], [2, 2], 128, torch.float16, 64),
    ([(i * 53) % 90 for i in range(70)], [(i * 5) % 3 for i in range(70)], 16, torch.bfloat16, 16),
]


@pytest.mark.parametrize("lens,q_lens,H,dt,page", PAGED_MLA_CASES)
def test_mla_varlen_paged(lens, q_lens, H, dt, page):
    x = workloads.make_inputs(spec_mla(lens, H, dt))
    vq = workloads.make_varlen_query(x, q_lens, seed=len(lens))
    check_paged(x, vq, page, f"mla varlen paged {lens[:6]} q {q_lens[:6]} H{H} {dt} page {page}")


def test_varlen_paged_without_mask_and_split():
    x = workloads.make_inputs(spec_gqa([40, 300, 7], 8, 2, 128, torch.float16))
    vq = workloads.make_varlen_query(x, [3, 20, 9], seed=3)
    check_paged(x, vq, 16, "gqa varlen paged, no mask, 64 workers", causal=False, num_workers=64)
    xm = workloads.make_inputs(spec_mla([40, 300, 7], 16, torch.bfloat16))
    vqm = workloads.make_varlen_query(xm, [3, 20, 9], seed=4)
    check_paged(xm, vqm, 64, "mla varlen paged, no mask, 64 workers", causal=False, num_workers=64)
