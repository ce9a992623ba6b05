"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on
identical seeded inputs.

Every case compares every output row, the five full-size workloads included
(in the benchmark's launch configuration: the library's default worker
count).  Outputs are pre-filled with NaN / +inf and surrounded by canaries
(tests/guard.py), so a row the kernels skip or a store out of bounds fails.
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


def odt(spec_or_dtype):
    dt = spec_or_dtype.torch_dtype if hasattr(spec_or_dtype, "torch_dtype") else spec_or_dtype
    return oracle.F16 if dt == torch.float16 else oracle.BF16


def ws_bytes(x: workloads.Inputs, num_workers=0):
    s = x.spec
    if s.kind == "mla":
        return zl().zl_decode_attn_mla_workspace_size(s.batch, s.num_q_heads, 512, 64, x.max_seqlen,
                                                      s.torch_dtype, num_workers)
    return zl().zl_decode_attn_workspace_size(s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim_k,
                                              x.max_seqlen, s.torch_dtype, num_workers)


def buffers(x: workloads.Inputs, num_workers=0, workspace=None):
    """Guarded out / lse (and a guarded workspace unless the caller brings one)."""
    s = x.spec
    return CallBuffers(s.batch, s.num_q_heads, s.head_dim_v, s.torch_dtype, DEV,
                       None if workspace is not None else ws_bytes(x, num_workers))


def run_gpu(x: workloads.Inputs, num_workers=0, workspace=None, where=""):
    s = x.spec
    cu = x.cu_seqlens.to(DEV)
    q = x.q.to(DEV)
    bufs = buffers(x, num_workers, workspace)
    kw = bufs.kwargs()
    if workspace is not None:
        kw["workspace"] = workspace
    if s.kind == "mla":
        out, lse = zl().zl_decode_attn_mla(q, x.latent.to(DEV), cu, x.max_seqlen, s.scale,
                                           num_workers=num_workers, **kw)
    else:
        out, lse = zl().zl_decode_attn_gqa(q, x.k.to(DEV), x.v.to(DEV), cu, x.max_seqlen, s.scale,
                                           num_workers=num_workers, **kw)
    torch.cuda.synchronize()
    bufs.check(where or s.name)
    return out, lse


def run_oracle(x: workloads.Inputs, pairs=None):
    s = x.spec
    cu = x.cu_seqlens.numpy()
    if s.kind == "mla":
        return oracle.mla_decode(x.bits("q"), x.bits("latent"), cu, s.scale, odt(s), pairs=pairs)
    return oracle.gqa_decode(x.bits("q"), x.bits("k"), x.bits("v"), cu, s.num_kv_heads, s.scale,
                             odt(s), pairs=pairs)


def check_full(x, where, **kw):
    out, lse = run_gpu(x, where=where, **kw)
    ro, rl = run_oracle(x)
    return gate(out, ro, x.spec.torch_dtype, lse, rl, where=where)


# ------------------------------------------------------------ the five workloads
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_every_row(cfg):
    """Each workload at its full size, every (sequence, head) row against the
    oracle, in the launch configuration the benchmark times."""
    spec = workloads.WORKLOADS[cfg]
    print(spec.name, flush=True)
    x = workloads.make_inputs(spec)
    st = check_full(x, spec.name)
    print(spec.name, st, flush=True)


# ------------------------------------------------------------- edge cases
GQA_EDGE = [
    # (batch lens, Hq, Hkv, D, dtype)
    ([1], 1, 1, 128, torch.float16),
    ([33, 1, 31, 32, 64, 65, 7], 8, 2, 128, torch.float16),
    ([5, 0, 130, 0, 2], 4, 4, 64, torch.bfloat16),
    ([0, 0, 0], 8, 1, 128, torch.float16),
    ([300, 17, 1000], 16, 1, 128, torch.bfloat16),
    ([129, 2, 70], 32, 1, 64, torch.float16),      # G = 32: two 16-head blocks
    ([96, 95, 97], 6, 2, 128, torch.bfloat16),     # G = 3 (padding heads)
    ([2000], 2, 1, 64, torch.float16),
    # more than 64 sequences: the lookups take the looped path instead of the
    # one-load boundary window; empty and one-token sequences mixed in
    ([(i * 37) % 50 for i in range(100)], 8, 2, 128, torch.float16),
    ([1] * 65, 4, 4, 64, torch.bfloat16),
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,dt", GQA_EDGE)
def test_gqa_edge_shapes(lens, Hq, Hkv, D, dt):
    spec = workloads.Spec("edge", "gqa", len(lens), Hq, Hkv, D, D, tuple(lens),
                          "f16" if dt == torch.float16 else "bf16", float(np.float32(1 / math.sqrt(D))), 7)
    x = workloads.make_inputs(spec)
    check_full(x, f"edge {lens} {Hq}/{Hkv} D{D} {dt}")


MLA_EDGE = [
    ([1, 33, 64], 16, torch.bfloat16),
    ([0, 257, 31], 16, torch.float16),
    ([100, 3], 8, torch.bfloat16),
    ([70, 0, 150], 32, torch.bfloat16),
    ([(i * 53) % 90 for i in range(80)], 16, torch.bfloat16),  # > 64 sequences
]


@pytest.mark.parametrize("lens,H,dt", MLA_EDGE)
def test_mla_edge_shapes(lens, H, dt):
    spec = workloads.Spec("mla-edge", "mla", len(lens), H, 1, 576, 512, tuple(lens),
                          "f16" if dt == torch.float16 else "bf16", float(np.float32(1 / math.sqrt(192))), 9)
    x = workloads.make_inputs(spec)
    check_full(x, f"mla edge {lens} H{H} {dt}")


@pytest.mark.parametrize("workers", [8, 16, 64, 256, 2048])
def test_any_worker_count_gives_the_same_attention(workers):
    """Invariance to how the batch is cut between workers (split-KV + combine)."""
    spec = workloads.with_shape(workloads.WORKLOADS[2], batch=6, lens=("uniform", 1, 3000))
    x = workloads.make_inputs(spec, seed=21)
    check_full(x, f"gqa workers={workers}", num_workers=workers)
    mspec = workloads.with_shape(workloads.WORKLOADS[5], batch=3, lens=("uniform", 1, 1500))
    xm = workloads.make_inputs(mspec, seed=22)
    check_full(xm, f"mla workers={workers}", num_workers=workers)


def test_peaked_scores():
    spec = workloads.with_shape(workloads.WORKLOADS[1], dtype="bf16")
    x = workloads.make_inputs(spec, q_mult=8.0)
    check_full(x, "peaked gqa")
    mspec = workloads.with_shape(workloads.WORKLOADS[5], batch=2, lens=(40, 300))
    xm = workloads.make_inputs(mspec, q_mult=4.0)
    check_full(xm, "peaked mla")


def test_repeated_calls_reuse_workspace_and_are_bitwise_deterministic():
    """Same inputs -> bitwise-identical output on every call; the workspace
    (no initialisation needed) carries nothing between calls."""
    spec = workloads.with_shape(workloads.WORKLOADS[3], batch=8, lens=("uniform", 100, 3000))
    x = workloads.make_inputs(spec, seed=31)
    B, H, D = x.q.shape
    ws = zl().new_workspace(zl().zl_decode_attn_workspace_size(B, H, 1, D, x.max_seqlen, x.q.dtype), DEV)
    ws.fill_(0xAB)  # garbage in the workspace must not matter
    outs = [run_gpu(x, workspace=ws)[0].clone() for _ in range(5)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    ro, rl = run_oracle(x)
    gate(outs[0], ro, spec.torch_dtype, where="repeat")
    # a different batch through the same workspace
    x2 = workloads.make_inputs(workloads.with_shape(spec, batch=3, lens=(5, 4000, 77)), seed=32)
    out2, lse2 = run_gpu(x2, workspace=ws)
    ro2, rl2 = run_oracle(x2)
    gate(out2, ro2, spec.torch_dtype, lse2, rl2, where="second batch")


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("S,Dv,dt", [(1, 128, torch.float16), (5, 128, torch.bfloat16), (13, 512, torch.bfloat16),
                                     (64, 64, torch.float16)])
def test_combine_entry_point(S, Dv, dt):
    rng = np.random.default_rng(S + Dv)
    B, H = 3, 4
    part_o = rng.standard_normal((S, B, H, Dv)).astype(np.float32)
    part_l = (rng.standard_normal((S, B, H)) * 3).astype(np.float32)
    part_l[rng.random((S, B, H)) < 0.2] = -np.inf     # some empty splits
    part_l[:, 0, 0] = -np.inf                          # one row with every split empty
    ro, rl = oracle.combine(part_o.astype(np.float64), part_l.astype(np.float64))
    bufs = CallBuffers(B, H, Dv, dt, DEV)
    out, lse = zl().zl_attn_combine(torch.from_numpy(part_o).to(DEV), torch.from_numpy(part_l).to(DEV),
                                    out_dtype=dt, **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check(f"combine S={S}")
    gate(out, ro, dt, lse, rl, where=f"combine S={S}")
    assert torch.all(out[0, 0] == 0)


def test_combine_of_oracle_partials_equals_unsplit_attention():
    spec = workloads.with_shape(workloads.WORKLOADS[2], batch=4, lens=(100, 257, 64, 1))
    x = workloads.make_inputs(spec, seed=41)
    S = 3
    B, Hq, D = x.q.shape
    po = np.zeros((S, B, Hq, D))
    pl = np.full((S, B, Hq), -np.inf)
    cu = x.cu_seqlens.numpy()
    for b in range(B):
        edges = np.linspace(0, cu[b + 1] - cu[b], S + 1).astype(int)
        for s in range(S):
            a, e = cu[b] + edges[s], cu[b] + edges[s + 1]
            sub = workloads.cu_from_lens([e - a]).numpy()
            o, l = oracle.gqa_decode(x.bits("q")[b:b + 1], x.bits("k")[a:e], x.bits("v")[a:e], sub,
                                     spec.num_kv_heads, spec.scale, oracle.F16)
            po[s, b], pl[s, b] = o[0], l[0]
    po32, pl32 = po.astype(np.float32), pl.astype(np.float32)
    bufs = CallBuffers(B, Hq, D, torch.float16, DEV)
    out, lse = zl().zl_attn_combine(torch.from_numpy(po32).to(DEV), torch.from_numpy(pl32).to(DEV),
                                    out_dtype=torch.float16, **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check("combine of partials")
    ro, rl = run_oracle(x)
    gate(out, ro, torch.float16, lse, rl, where="combine of partials")


# ------------------------------------------------------------ paged caches
def run_gpu_paged(x: workloads.Inputs, p: workloads.PagedInputs, num_workers=0, where=""):
    s = x.spec
    cu = x.cu_seqlens.to(DEV)
    q = x.q.to(DEV)
    bt = p.block_table.to(DEV)
    bufs = buffers(x, num_workers)
    if s.kind == "mla":
        out, lse = zl().zl_decode_attn_mla_paged(q, p.kv_pages.to(DEV), bt, cu, x.max_seqlen, s.scale,
                                                 num_workers=num_workers, **bufs.kwargs())
    else:
        out, lse = zl().zl_decode_attn_gqa_paged(q, p.k_pages.to(DEV), p.v_pages.to(DEV), bt, cu,
                                                 x.max_seqlen, s.scale, num_workers=num_workers,
                                                 **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check(where or f"paged {s.name}")
    return out, lse


def u16(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def run_oracle_paged(x: workloads.Inputs, p: workloads.PagedInputs, pairs=None):
    s = x.spec
    cu = x.cu_seqlens.numpy()
    bt = p.block_table.numpy()
    if s.kind == "mla":
        return oracle.mla_decode_paged(x.bits("q"), u16(p.kv_pages), bt, cu, s.scale, odt(s), pairs=pairs)
    return oracle.gqa_decode_paged(x.bits("q"), u16(p.k_pages), u16(p.v_pages), bt, cu, s.num_kv_heads, s.scale, odt(s), pairs=pairs)


PAGED_GQA = [
    # (batch lens, Hq, Hkv, D, dtype, page size)
    ([33, 1, 31, 32, 64, 65, 7], 8, 2, 128, torch.float16, 16),
    ([33, 1, 31, 32, 64, 65, 7], 8, 2, 128, torch.float16, 64),
    ([5, 0, 130, 0, 2], 4, 4, 64, torch.bfloat16, 32),
    ([300, 17, 1000], 16, 1, 128, torch.bfloat16, 256),
    ([129, 2, 70], 32, 1, 64, torch.float16, 16),
    ([(i * 37) % 50 for i in range(100)], 8, 2, 128, torch.float16, 16),   # > 64 sequences
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,dt,ps", PAGED_GQA)
def test_gqa_paged(lens, Hq, Hkv, D, dt, ps):
    spec = workloads.Spec("paged", "gqa", len(lens), Hq, Hkv, D, D, tuple(lens),
                          "f16" if dt == torch.float16 else "bf16", float(np.float32(1 / math.sqrt(D))), 7)
    x = workloads.make_inputs(spec)
    p = workloads.make_paged(x, ps, seed=len(lens) + ps)
    where = f"paged gqa {lens} {Hq}/{Hkv} D{D} {dt} ps{ps}"
    print(where, flush=True)
    out, lse = run_gpu_paged(x, p, where=where)
    ro, rl = run_oracle_paged(x, p)
    gate(out, ro, dt, lse, rl, where=where)
    # the page layout changes where rows live, not the arithmetic: the packed
    # path on the same rows gives the same bits
    po, pl = run_gpu(x)
    assert torch.equal(out, po) and torch.equal(lse, pl)


PAGED_MLA = [
    ([0, 257, 31], 16, torch.float16, 64),
    ([70, 0, 150], 32, torch.bfloat16, 16),
    ([1, 33, 64], 16, torch.bfloat16, 128),
    ([(i * 53) % 90 for i in range(80)], 16, torch.bfloat16, 16),   # > 64 sequences
]


@pytest.mark.parametrize("lens,H,dt,ps", PAGED_MLA)
def test_mla_paged(lens, H, dt, ps):
    spec = workloads.Spec("paged-mla", "mla", len(lens), H, 1, 576, 512, tuple(lens),
                          "f16" if dt == torch.float16 else "bf16", float(np.float32(1 / math.sqrt(192))), 9)
    x = workloads.make_inputs(spec)
    p = workloads.make_paged(x, ps, seed=len(lens) + ps)
    where = f"paged mla {lens} H{H} {dt} ps{ps}"
    print(where, flush=True)
    out, lse = run_gpu_paged(x, p, where=where)
    ro, rl = run_oracle_paged(x, p)
    gate(out, ro, dt, lse, rl, where=where)
    po, pl = run_gpu(x)
    assert torch.equal(out, po) and torch.equal(lse, pl)


@pytest.mark.parametrize("cfg,ps", [(2, 16), (3, 32), (4, 256), (5, 64)])
def test_full_size_paged_every_row(cfg, ps):
    """Full-size workloads over shuffled page pools: every row against the
    oracle on the gathered rows, and bitwise equal to the packed path."""
    spec = workloads.WORKLOADS[cfg]
    where = f"paged {spec.name}, {ps}-token pages"
    print(where, flush=True)
    x = workloads.make_inputs(spec)
    p = workloads.make_paged(x, ps, seed=cfg)
    out, lse = run_gpu_paged(x, p, where=where)
    ro, rl = run_oracle_paged(x, p)
    gate(out, ro, spec.torch_dtype, lse, rl, where=where)
    po, pl = run_gpu(x)
    assert torch.equal(out, po) and torch.equal(lse, pl)
