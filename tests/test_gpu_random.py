"""GPU parity on seeded random shapes: every decode-family entry point (one or
several new tokens, packed or paged caches, GQA or MLA, f16 or bf16, causal
or not, library-chosen or forced worker counts) against the fp64 oracle on
identical inputs.  The cases are drawn from a fixed seed, so a failure names
a reproducible case; they complement the hand-picked edge cases with shapes
nobody chose.  ZL_RANDOM_CASES and ZL_RANDOM_PREFILL_CASES widen the sweep
(case i is the same draw whatever the count).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.guard import CallBuffers
from tests.parity import gate

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = int(os.environ.get("ZL_RANDOM_CASES", "200"))
N_PREFILL_CASES = int(os.environ.get("ZL_RANDOM_PREFILL_CASES", "100"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_amd as zl
    zl.library()
    yield


def draw_case(i: int) -> dict:
    """Case i of the sweep (pure function of i)."""
    r = np.random.default_rng(1000 + i)
    kind = "mla" if r.random() < 0.35 else "gqa"
    dt = torch.float16 if r.random() < 0.5 else torch.bfloat16
    B = int(r.choice([1, 2, 3, 7, 16, 33, 70]))
    lens = [int(v) for v in r.integers(0, 700, size=B)]
    if r.random() < 0.2:
        lens[int(r.integers(0, B))] = 0
    multi = r.random() < 0.5
    q_lens = [int(v) for v in r.integers(0, 6, size=B)] if multi else None
    paged = int(r.choice([0, 16, 32, 64, 128, 256]))
    workers = int(r.choice([0, 0, 8, 64, 256, 1024]))
    causal = bool(r.random() < 0.8)
    if kind == "mla":
        H = int(r.choice([8, 16, 32, 64, 128]))
        case = dict(kind=kind, H=H, Hkv=1, D=576)
    else:
        D = int(r.choice([64, 128]))
        Hkv = int(r.choice([1, 2, 4, 8]))
        G = int(r.choice([1, 2, 3, 4, 8, 16, 32]))
        case = dict(kind=kind, H=Hkv * G, Hkv=Hkv, D=D)
    # Keep the oracle's work (new tokens x cached rows x heads x dims) to a
    # few seconds: shorten the lengths if the draw is large.
    dims = 1088 if kind == "mla" else 2 * case["D"]
    work = sum(max(q, 1) * L for q, L in zip(q_lens or [1] * B, lens)) * case["H"] * dims
    if work > 3e9:
        f = 3e9 / work
        lens = [int(L * f) for L in lens]
    case.update(dt=dt, lens=lens, q_lens=q_lens, paged=paged, workers=workers, causal=causal, seed=i)
    return case


def spec_of(c) -> workloads.Spec:
    dts = "f16" if c["dt"] == torch.float16 else "bf16"
    if c["kind"] == "mla":
        return workloads.Spec("random-mla", "mla", len(c["lens"]), c["H"], 1, 576, 512, tuple(c["lens"]), dts,
                              float(np.float32(1 / math.sqrt(192))), c["seed"])
    return workloads.Spec("random-gqa", "gqa", len(c["lens"]), c["H"], c["Hkv"], c["D"], c["D"], tuple(c["lens"]),
                          dts, float(np.float32(1 / math.sqrt(c["D"]))), c["seed"])


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    import mla_attention_amd as zl
    c = draw_case(i)
    s = spec_of(c)
    x = workloads.make_inputs(s)
    q_lens = c["q_lens"] if c["q_lens"] is not None else [1] * s.batch
    if c["q_lens"] is not None:
        vq = workloads.make_varlen_query(x, q_lens, seed=i)
        q, cu_q = vq.q, vq.cu_q
    else:
        q, cu_q = x.q, workloads.cu_from_lens(q_lens)
    where = (f"case {i}: {c['kind']} {c['dt']} B={s.batch} H={s.num_q_heads}/{s.num_kv_heads} D={s.head_dim_k} "
             f"lens={c['lens'][:8]} q_lens={q_lens[:8] if c['q_lens'] is not None else 'decode'} "
             f"paged={c['paged']} workers={c['workers']} causal={c['causal']}")
    print(where, flush=True)
    if c["q_lens"] is not None and sum(q_lens) == 0:
        pytest.skip("no new tokens drawn")
    if c["q_lens"] is None and not c["causal"]:
        c["causal"] = True  # decode has no mask switch: one new token sees its whole cache

    dq, ck = q.to(DEV), x.cu_seqlens.to(DEV)
    if s.kind == "mla":
        ws = zl.zl_decode_attn_mla_workspace_size(s.batch, s.num_q_heads, 512, 64, x.max_seqlen, s.torch_dtype,
                                                  c["workers"])
    else:
        ws = zl.zl_decode_attn_workspace_size(s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim_k, x.max_seqlen,
                                              s.torch_dtype, c["workers"])
    bufs = CallBuffers(q.shape[0], s.num_q_heads, s.head_dim_v, s.torch_dtype, DEV, ws)
    kw = dict(num_workers=c["workers"], **bufs.kwargs())
    px = workloads.make_paged(x, c["paged"], seed=i) if c["paged"] else None
    bt = px.block_table.to(DEV) if px else None
    mla = s.kind == "mla"
    if c["q_lens"] is not None:
        dcq = cu_q.to(DEV)
        if mla and px:
            out, lse = zl.zl_attn_varlen_mla_paged(dq, px.kv_pages.to(DEV), bt, dcq, ck, x.max_seqlen, s.scale,
                                                   causal=c["causal"], **kw)
        elif mla:
            out, lse = zl.zl_attn_varlen_mla(dq, x.latent.to(DEV), dcq, ck, x.max_seqlen, s.scale,
                                             causal=c["causal"], **kw)
        elif px:
            out, lse = zl.zl_attn_varlen_gqa_paged(dq, px.k_pages.to(DEV), px.v_pages.to(DEV), bt, dcq, ck,
                                                   x.max_seqlen, s.scale, causal=c["causal"], **kw)
        else:
            out, lse = zl.zl_attn_varlen_gqa(dq, x.k.to(DEV), x.v.to(DEV), dcq, ck, x.max_seqlen, s.scale,
                                             causal=c["causal"], **kw)
    else:
        if mla and px:
            out, lse = zl.zl_decode_attn_mla_paged(dq, px.kv_pages.to(DEV), bt, ck, x.max_seqlen, s.scale, **kw)
        elif mla:
            out, lse = zl.zl_decode_attn_mla(dq, x.latent.to(DEV), ck, x.max_seqlen, s.scale, **kw)
        elif px:
            out, lse = zl.zl_decode_attn_gqa_paged(dq, px.k_pages.to(DEV), px.v_pages.to(DEV), bt, ck,
                                                   x.max_seqlen, s.scale, **kw)
        else:
            out, lse = zl.zl_decode_attn_gqa(dq, x.k.to(DEV), x.v.to(DEV), ck, x.max_seqlen, s.scale, **kw)
    torch.cuda.synchronize()
    bufs.check(where)

    # The oracle on the packed rows (paged pools hold the same rows).
    qb = q.contiguous().view(torch.int16).numpy().view(np.uint16)
    odt = oracle.F16 if c["dt"] == torch.float16 else oracle.BF16
    cqn, ckn = cu_q.numpy(), x.cu_seqlens.numpy()
    if mla:
        ro, rl = oracle.mla_varlen(qb, x.bits("latent"), cqn, ckn, s.scale, odt, causal=c["causal"])
    else:
        ro, rl = oracle.gqa_varlen(qb, x.bits("k"), x.bits("v"), cqn, ckn, s.num_kv_heads, s.scale, odt,
                                   causal=c["causal"])
    gate(out, ro, c["dt"], lse, rl, where=where)


def draw_prefill_case(i: int) -> dict:
    """Prefill case i: runs of new tokens (whole prompts or chunks after a
    cached prefix), drawn from a fixed seed."""
    r = np.random.default_rng(5000 + i)
    B = int(r.choice([1, 2, 3, 5, 9]))
    D = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 3, 4, 8, 16]))
    q_lens, lens = [], []
    for _ in range(B):
        nq = int(r.integers(0, 400))
        prefix = int(r.integers(0, 400)) if r.random() < 0.5 else 0
        q_lens.append(nq)
        lens.append(nq + prefix)
    # A few draws with more new tokens than cached rows (leading tokens see none).
    if r.random() < 0.15:
        q_lens[0] = lens[0] + int(r.integers(1, 20))
    work = sum(q * L for q, L in zip(q_lens, lens)) * Hkv * G * 2 * D
    if work > 1.5e9:
        f = math.sqrt(1.5e9 / work)
        q_lens = [int(q * f) for q in q_lens]
        lens = [max(int(L * f), q) for q, L in zip(q_lens, lens)]
    dt = torch.float16 if r.random() < 0.5 else torch.bfloat16
    return dict(B=B, D=D, Hkv=Hkv, H=Hkv * G, lens=lens, q_lens=q_lens, dt=dt, causal=bool(r.random() < 0.8),
                seed=100 + i)


@pytest.mark.parametrize("i", range(N_PREFILL_CASES))
def test_random_prefill_case(i):
    import mla_attention_amd as zl
    c = draw_prefill_case(i)
    spec = workloads.Spec("random-prefill", "gqa", c["B"], c["H"], c["Hkv"], c["D"], c["D"], tuple(c["lens"]),
                          "f16" if c["dt"] == torch.float16 else "bf16", float(np.float32(1 / math.sqrt(c["D"]))),
                          c["seed"])
    where = (f"prefill case {i}: {c['dt']} H={c['H']}/{c['Hkv']} D={c['D']} lens={c['lens']} q_lens={c['q_lens']} "
             f"causal={c['causal']}")
    print(where, flush=True)
    if sum(c["q_lens"]) == 0:
        pytest.skip("no new tokens drawn")
    x = workloads.make_inputs(spec)
    vq = workloads.make_varlen_query(x, c["q_lens"], seed=c["seed"])
    bufs = CallBuffers(vq.total_q, spec.num_q_heads, spec.head_dim_v, spec.torch_dtype, DEV)
    out, lse = zl.zl_attn_prefill_gqa(vq.q.to(DEV), x.k.to(DEV), x.v.to(DEV), vq.cu_q.to(DEV), x.cu_seqlens.to(DEV),
                                      x.max_seqlen, spec.scale, causal=c["causal"], **bufs.kwargs())
    torch.cuda.synchronize()
    bufs.check(where)
    qb = vq.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    odt = oracle.F16 if c["dt"] == torch.float16 else oracle.BF16
    ro, rl = oracle.gqa_varlen(qb, x.bits("k"), x.bits("v"), vq.cu_q.numpy(), x.cu_seqlens.numpy(), c["Hkv"],
                               spec.scale, odt, causal=c["causal"])
    gate(out, ro, c["dt"], lse, rl, where=where)
