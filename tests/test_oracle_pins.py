"""Pins of the fp64 oracle against things other than itself.

The pages print no worked example and no formula, so every pin here is a
closed form, a reduction to a library routine (torch's scaled-dot-product
attention and logsumexp in float64), an invariant of softmax attention, or a
brute-force evaluation by a different method.  They are chosen so that a
plausible slip in the oracle -- a dropped scale, a wrong head mapping, a
transposed K or V, a missing normalisation, a wrong log base, a wrong combine
weight -- fails at least one of them (tests/test_oracle_mutants.py checks
exactly that by planting such slips).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rand16(shape, dtype, gen, lo=None, hi=None):
    """Random 16-bit tensor; with lo/hi, small integers (exact in 16 bits)."""
    if lo is not None:
        return torch.randint(lo, hi + 1, shape, generator=gen).to(dtype)
    return torch.randn(shape, generator=gen).to(dtype)


def sdpa_reference(q, k, v, cu, num_kv_heads, scale):
    """torch.nn.functional.scaled_dot_product_attention in float64, per sequence,
    with key/value heads repeated to the query heads (repeat_interleave)."""
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    qd = q.to(torch.float64)
    kd = k.to(torch.float64)
    vd = v.to(torch.float64)
    outs, lses = [], []
    for b in range(B):
        s, e = int(cu[b]), int(cu[b + 1])
        kb = kd[s:e].permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, D]
        vb = vd[s:e].permute(1, 0, 2).repeat_interleave(G, dim=0)
        qb = qd[b].unsqueeze(1)                                     # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, scale=scale)
        scores = (qb @ kb.transpose(1, 2)).squeeze(1) * scale       # [Hq, L]
        outs.append(o.squeeze(1))
        lses.append(torch.logsumexp(scores, dim=-1))
    return torch.stack(outs).numpy(), torch.stack(lses).numpy()


def run_gqa(q, k, v, cu, num_kv_heads, scale, dtype):
    dt = oracle.F16 if dtype == torch.float16 else oracle.BF16
    return oracle.gqa_decode(bits(q), bits(k), bits(v), np.asarray(cu, dtype=np.int32),
                             num_kv_heads, scale, dt)


# ---------------------------------------------------------------- P11 decoders
@pytest.mark.parametrize("dtype,code", [(torch.float16, oracle.F16), (torch.bfloat16, oracle.BF16)])
def test_p11_decoders_all_patterns(dtype, code):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode(pats, code)
    ref = torch.from_numpy(pats.view(np.int16).copy()).view(dtype).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


# ------------------------------------------------------- library-routine pin
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 64), (4, 4, 32), (6, 1, 16), (16, 1, 72)])
def test_matches_torch_sdpa_float64(dtype, Hq, Hkv, D):
    gen = torch.Generator().manual_seed(100 + Hq + D)
    lens = [1, 5, 33, 17]
    cu = workloads.cu_from_lens(lens)
    T = int(cu[-1])
    q = rand16((4, Hq, D), dtype, gen)
    k = rand16((T, Hkv, D), dtype, gen)
    v = rand16((T, Hkv, D), dtype, gen)
    scale = float(np.float32(0.37))
    out, lse = run_gqa(q, k, v, cu, Hkv, scale, dtype)
    ro, rl = sdpa_reference(q, k, v, cu, Hkv, scale)
    np.testing.assert_allclose(out, ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_config1_matches_torch_sdpa():
    x = workloads.make_inputs(workloads.WORKLOADS[1])
    out, lse = run_gqa(x.q, x.k, x.v, x.cu_seqlens, 2, x.spec.scale, torch.float16)
    ro, rl = sdpa_reference(x.q, x.k, x.v, x.cu_seqlens, 2, x.spec.scale)
    np.testing.assert_allclose(out, ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- P1 q = 0
@pytest.mark.parametrize("use_scale_zero", [False, True])
def test_p1_uniform_weights_give_mean_of_v(use_scale_zero):
    gen = torch.Generator().manual_seed(1)
    lens = [3, 10, 1, 64]
    cu = workloads.cu_from_lens(lens)
    T = int(cu[-1])
    q = rand16((4, 4, 32), torch.float16, gen)
    if not use_scale_zero:
        q = torch.zeros_like(q)
    k = rand16((T, 2, 32), torch.float16, gen)
    v = rand16((T, 2, 32), torch.float16, gen)
    out, lse = run_gqa(q, k, v, cu, 2, 0.0 if use_scale_zero else 0.25, torch.float16)
    vd = v.to(torch.float64).numpy()
    for b, L in enumerate(lens):
        s = int(cu[b])
        for h in range(4):
            np.testing.assert_allclose(out[b, h], vd[s:s + L, h // 2].mean(axis=0), rtol=1e-14, atol=1e-15)
            assert lse[b, h] == pytest.approx(math.log(L), abs=1e-14)


# ---------------------------------------------------------------- P2 L = 1
def test_p2_single_token_returns_its_value():
    gen = torch.Generator().manual_seed(2)
    cu = workloads.cu_from_lens([1, 1])
    q = rand16((2, 2, 16), torch.bfloat16, gen)
    k = rand16((2, 1, 16), torch.bfloat16, gen)
    v = rand16((2, 1, 16), torch.bfloat16, gen)
    out, lse = run_gqa(q, k, v, cu, 1, 0.5, torch.bfloat16)
    qd, kd, vd = (t.to(torch.float64).numpy() for t in (q, k, v))
    for b in range(2):
        for h in range(2):
            assert np.array_equal(out[b, h], vd[b, 0])
            assert lse[b, h] == pytest.approx(0.5 * float(qd[b, h] @ kd[b, 0]), rel=1e-15, abs=1e-15)


# ----------------------------------------------------------- empty sequence
def test_empty_sequence_gives_zero_and_minus_inf():
    gen = torch.Generator().manual_seed(3)
    cu = workloads.cu_from_lens([0, 4, 0])
    q = rand16((3, 2, 8), torch.float16, gen)
    k = rand16((4, 1, 8), torch.float16, gen)
    v = rand16((4, 1, 8), torch.float16, gen)
    out, lse = run_gqa(q, k, v, cu, 1, 0.3, torch.float16)
    for b in (0, 2):
        assert np.all(out[b] == 0.0)
        assert np.all(np.isneginf(lse[b]))
    assert np.all(np.isfinite(out[1]))


# ------------------------------------------------- P3 shift of every score
def test_p3_constant_added_to_scores():
    """K' = K + 1 u^T adds scale * q.u to every score of a row: out is unchanged
    and lse moves by exactly that constant.  Integer entries keep K' exact."""
    gen = torch.Generator().manual_seed(4)
    lens = [7, 20]
    cu = workloads.cu_from_lens(lens)
    T = int(cu[-1])
    q = rand16((2, 4, 16), torch.float16, gen, -3, 3)
    k = rand16((T, 2, 16), torch.float16, gen, -3, 3)
    v = rand16((T, 2, 16), torch.float16, gen)
    u = torch.randint(-2, 3, (2, 16), generator=gen).to(torch.float16)
    scale = 0.125
    out0, lse0 = run_gqa(q, k, v, cu, 2, scale, torch.float16)
    out1, lse1 = run_gqa(q, k + u.unsqueeze(0), v, cu, 2, scale, torch.float16)
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-14)
    qd, ud = q.to(torch.float64).numpy(), u.to(torch.float64).numpy()
    for b in range(2):
        for h in range(4):
            assert lse1[b, h] - lse0[b, h] == pytest.approx(scale * float(qd[b, h] @ ud[h // 2]), abs=1e-12)


# ------------------------------------ P4 brute force, different method
def test_p4_naive_softmax_long_double_bruteforce():
    """exp(s_i)/sum_j exp(s_j) without max subtraction, in numpy longdouble,
    scores kept small so nothing overflows; a different evaluation order."""
    gen = torch.Generator().manual_seed(5)
    lens = [2, 9, 31]
    cu = workloads.cu_from_lens(lens)
    T = int(cu[-1])
    q = rand16((3, 3, 12), torch.bfloat16, gen)
    k = rand16((T, 3, 12), torch.bfloat16, gen)
    v = rand16((T, 3, 12), torch.bfloat16, gen)
    scale = 0.7
    out, lse = run_gqa(q, k, v, cu, 3, scale, torch.bfloat16)
    qd, kd, vd = (np.asarray(t.to(torch.float64).numpy(), dtype=np.longdouble) for t in (q, k, v))
    for b in range(3):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for h in range(3):
            scores = np.array([sum(qd[b, h, d] * kd[t, h, d] for d in range(12)) for t in range(s0, s1)],
                              dtype=np.longdouble) * np.longdouble(scale)
            assert np.all(np.abs(scores) < 40)
            e = np.exp(scores)
            z = e.sum()
            ref = sum(e[i] * vd[s0 + i, h] for i in range(s1 - s0)) / z
            np.testing.assert_allclose(out[b, h], ref.astype(np.float64), rtol=1e-13, atol=1e-14)
            assert lse[b, h] == pytest.approx(float(np.log(z)), abs=1e-13)


# ------------------------------------------------------ P5 token permutation
def test_p5_token_order_does_not_matter():
    gen = torch.Generator().manual_seed(6)
    L = 50
    cu = workloads.cu_from_lens([L])
    q = rand16((1, 4, 32), torch.float16, gen)
    k = rand16((L, 1, 32), torch.float16, gen)
    v = rand16((L, 1, 32), torch.float16, gen)
    perm = torch.randperm(L, generator=gen)
    out0, lse0 = run_gqa(q, k, v, cu, 1, 0.2, torch.float16)
    out1, lse1 = run_gqa(q, k[perm], v[perm], cu, 1, 0.2, torch.float16)
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse1, lse0, rtol=1e-14)


# ----------------------------------------------------------- P6 duplication
def test_p6_duplicating_every_row_adds_ln2():
    gen = torch.Generator().manual_seed(7)
    L = 23
    q = rand16((1, 2, 16), torch.bfloat16, gen)
    k = rand16((L, 2, 16), torch.bfloat16, gen)
    v = rand16((L, 2, 16), torch.bfloat16, gen)
    out0, lse0 = run_gqa(q, k, v, workloads.cu_from_lens([L]), 2, 0.4, torch.bfloat16)
    out1, lse1 = run_gqa(q, torch.cat([k, k]), torch.cat([v, v]), workloads.cu_from_lens([2 * L]), 2,
                         0.4, torch.bfloat16)
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse1 - lse0, math.log(2.0), atol=1e-13)


# ------------------------------------------------------ P7 linearity in V
def test_p7_affine_in_v_and_constant_v():
    gen = torch.Generator().manual_seed(8)
    lens = [5, 40]
    cu = workloads.cu_from_lens(lens)
    T = int(cu[-1])
    q = rand16((2, 2, 16), torch.float16, gen)
    k = rand16((T, 1, 16), torch.float16, gen)
    v = rand16((T, 1, 16), torch.float16, gen, -8, 8)
    out0, _ = run_gqa(q, k, v, cu, 1, 0.3, torch.float16)
    out1, _ = run_gqa(q, k, 2 * v + 1, cu, 1, 0.3, torch.float16)  # exact in fp16
    np.testing.assert_allclose(out1, 2 * out0 + 1, rtol=1e-13, atol=1e-13)
    const = torch.full((T, 1, 16), 0.75, dtype=torch.float16)
    out2, _ = run_gqa(q, k, const, cu, 1, 0.3, torch.float16)
    np.testing.assert_allclose(out2, 0.75, rtol=1e-14)  # exact up to fp64 summation rounding


# ------------------------------------------------------ P8 GQA head mapping
def test_p8_gqa_equals_mha_on_repeated_kv_heads():
    gen = torch.Generator().manual_seed(9)
    lens = [12, 3, 30]
    cu = workloads.cu_from_lens(lens)
    T = int(cu[-1])
    Hq, Hkv, D = 8, 2, 16
    q = rand16((3, Hq, D), torch.float16, gen)
    k = rand16((T, Hkv, D), torch.float16, gen)
    v = rand16((T, Hkv, D), torch.float16, gen)
    out_g, lse_g = run_gqa(q, k, v, cu, Hkv, 0.25, torch.float16)
    krep = k.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    vrep = v.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    out_m, lse_m = run_gqa(q, krep, vrep, cu, Hq, 0.25, torch.float16)
    assert np.array_equal(out_g, out_m) and np.array_equal(lse_g, lse_m)
    # and each group of query heads really shares one key/value head
    for h in range(Hq):
        out_1, _ = run_gqa(q[:, h:h + 1].contiguous(), k[:, h // (Hq // Hkv):h // (Hq // Hkv) + 1].contiguous(),
                           v[:, h // (Hq // Hkv):h // (Hq // Hkv) + 1].contiguous(), cu, 1, 0.25, torch.float16)
        assert np.array_equal(out_1[:, 0], out_g[:, h])


# ----------------------------------------------------------- P9 combine
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p9_combine_of_any_partition_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    gen = torch.Generator().manual_seed(seed)
    lens = [int(x) for x in rng.integers(1, 90, size=5)]
    cu = workloads.cu_from_lens(lens)
    T = int(cu[-1])
    Hq, Hkv, D = 4, 2, 24
    q = rand16((5, Hq, D), torch.bfloat16, gen)
    k = rand16((T, Hkv, D), torch.bfloat16, gen)
    v = rand16((T, Hkv, D), torch.bfloat16, gen)
    full_o, full_l = run_gqa(q, k, v, cu, Hkv, 0.3, torch.bfloat16)
    S = 4
    part_o = np.zeros((S, 5, Hq, D))
    part_l = np.full((S, 5, Hq), -np.inf)
    for b, L in enumerate(lens):
        cuts = np.sort(rng.integers(0, L + 1, size=S - 1))     # empty splits allowed
        edges = [0, *cuts.tolist(), L]
        for s in range(S):
            a, e = edges[s], edges[s + 1]
            sub_cu = workloads.cu_from_lens([e - a])
            o, l = run_gqa(q[b:b + 1].contiguous(), k[int(cu[b]) + a:int(cu[b]) + e].contiguous(),
                           v[int(cu[b]) + a:int(cu[b]) + e].contiguous(), sub_cu, Hkv, 0.3, torch.bfloat16)
            part_o[s, b], part_l[s, b] = o[0], l[0]
    comb_o, comb_l = oracle.combine(part_o, part_l)
    np.testing.assert_allclose(comb_o, full_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(comb_l, full_l, rtol=1e-13, atol=1e-13)


def test_combine_closed_forms():
    # two splits with equal lse: plain average, lse + ln 2
    po = np.array([[[1.0, -2.0]], [[3.0, 4.0]]])
    pl = np.array([[0.5], [0.5]])
    o, l = oracle.combine(po, pl)
    np.testing.assert_allclose(o, [[2.0, 1.0]], rtol=1e-15)
    assert l[0] == pytest.approx(0.5 + math.log(2), abs=1e-15)
    # weights e^a : e^b
    pl = np.array([[0.0], [math.log(3.0)]])
    o, l = oracle.combine(po, pl)
    np.testing.assert_allclose(o, [[(1 + 3 * 3) / 4, (-2 + 4 * 3) / 4]], rtol=1e-14)
    assert l[0] == pytest.approx(math.log(4.0), abs=1e-15)
    # an empty split (-inf, garbage payload) is ignored; all empty -> 0, -inf
    po = np.array([[[np.nan, np.nan]], [[3.0, 4.0]]])
    pl = np.array([[-np.inf], [1.25]])
    o, l = oracle.combine(po, pl)
    np.testing.assert_allclose(o, [[3.0, 4.0]])
    assert l[0] == 1.25
    o, l = oracle.combine(np.zeros((2, 1, 2)), np.full((2, 1), -np.inf))
    assert np.all(o == 0) and np.isneginf(l[0])


# --------------------------------------------------------------- P10 MLA
def test_p10_mla_equals_gqa_with_materialised_value_copy():
    gen = torch.Generator().manual_seed(10)
    lens = [9, 40, 1]
    cu = workloads.cu_from_lens(lens)
    T = int(cu[-1])
    q = rand16((3, 16, 576), torch.bfloat16, gen)
    c = rand16((T, 576), torch.bfloat16, gen)
    scale = float(np.float32(1 / math.sqrt(192)))
    out, lse = oracle.mla_decode(bits(q), bits(c), cu.numpy(), scale, oracle.BF16)
    kmat = c.unsqueeze(1).contiguous()                   # [T, 1, 576]
    vmat = c[:, :512].clone().unsqueeze(1).contiguous()  # separate copy of cols 0..511
    out2, lse2 = oracle.decode_attn(bits(q), bits(kmat), bits(vmat), cu.numpy(), 1, 576, 512, 576, 512,
                                    scale, oracle.BF16)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    ro, rl = sdpa_reference(q, kmat, torch.nn.functional.pad(vmat, (0, 64)), cu, 1, scale)
    np.testing.assert_allclose(out, ro[..., :512], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_p10_absorbed_equals_unabsorbed_attention():
    """With random up-projections W_UK, W_UV (per head), attention over the
    un-absorbed keys k = [W_UK c ; rope] and values v = W_UV c equals W_UV
    applied to the absorbed-form output (associativity)."""
    gen = torch.Generator().manual_seed(11)
    H, R, P, Dn = 4, 512, 64, 128
    L = 37
    cu = workloads.cu_from_lens([L])
    c = rand16((L, R + P), torch.bfloat16, gen)
    q_abs = rand16((1, H, R + P), torch.bfloat16, gen)
    scale = float(np.float32(1 / math.sqrt(192)))
    out, lse = oracle.mla_decode(bits(q_abs), bits(c), cu.numpy(), scale, oracle.BF16)
    g64 = torch.Generator().manual_seed(12)
    cd = c.to(torch.float64)
    qa = q_abs.to(torch.float64)[0]
    for h in range(H):
        q_nope = torch.randn(Dn, generator=g64, dtype=torch.float64)
        # W_UK with W_UK^T q_nope = q_abs[:512] exactly (up to fp64 rounding)
        W = torch.randn(Dn, R, generator=g64, dtype=torch.float64)
        W = W - torch.outer(q_nope, q_nope @ W) / (q_nope @ q_nope) + torch.outer(q_nope, qa[h, :R]) / (q_nope @ q_nope)
        W_UV = torch.randn(Dn, R, generator=g64, dtype=torch.float64)
        keys = torch.cat([cd[:, :R] @ W.T, cd[:, R:]], dim=1)          # [L, Dn+P]
        vals = cd[:, :R] @ W_UV.T                                      # [L, Dn]
        qq = torch.cat([q_nope, qa[h, R:]])
        ref = torch.nn.functional.scaled_dot_product_attention(qq.view(1, 1, -1), keys.unsqueeze(0),
                                                               vals.unsqueeze(0), scale=scale)
        np.testing.assert_allclose((W_UV @ torch.from_numpy(out[0, h])).numpy(), ref.view(-1).numpy(),
                                   rtol=1e-9, atol=1e-10)
        np.testing.assert_allclose(lse[0, h], torch.logsumexp(scale * keys @ qq, 0).item(), atol=1e-10)


# --------------------------------------------------- P12 one-hot dominance
def test_p12_dominant_key_selects_its_value():
    gen = torch.Generator().manual_seed(13)
    L, D = 16, 32
    k = rand16((L, 1, D), torch.float16, gen)
    v = rand16((L, 1, D), torch.float16, gen)
    j = 11
    q = (k[j, 0].to(torch.float32) * 8).to(torch.float16).view(1, 1, D)
    out, lse = run_gqa(q, k, v, workloads.cu_from_lens([L]), 1, 1.0, torch.float16)
    kd = k.to(torch.float64).numpy()[:, 0]
    s = kd @ q.to(torch.float64).numpy()[0, 0]
    assert np.sort(s)[-1] - np.sort(s)[-2] > 40     # separation >> 40 nats
    np.testing.assert_allclose(out[0, 0], v.to(torch.float64).numpy()[j, 0], rtol=0, atol=1e-15)
    assert lse[0, 0] == pytest.approx(s[j], rel=1e-15)


# ------------------------------------------- hand-derived worked examples
def _golden_cases():
    path = os.path.join(GOLDEN, "worked_examples.txt")
    cases, cur = [], None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, val = line.partition("=")
            key, val = key.strip(), val.strip()
            if key == "case":
                cur = {"name": val}
                cases.append(cur)
            else:
                cur[key] = val
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_worked_examples(case):
    ev = lambda s: eval(s, {"__builtins__": {}}, {"e": math.e, "ln": math.log, "exp": math.exp,
                                                  "sqrt": math.sqrt})
    q = torch.tensor(ev(case["q"]), dtype=torch.float16).view(1, 1, -1)
    k = torch.tensor(ev(case["k"]), dtype=torch.float16)
    k = k.view(k.shape[0], 1, -1)
    v = torch.tensor(ev(case["v"]), dtype=torch.float16)
    v = v.view(v.shape[0], 1, -1)
    scale = float(ev(case["scale"]))
    out, lse = run_gqa(q, k, v, workloads.cu_from_lens([k.shape[0]]), 1, scale, torch.float16)
    np.testing.assert_allclose(out[0, 0], ev(case["out"]), rtol=1e-14, atol=1e-15)
    assert lse[0, 0] == pytest.approx(ev(case["lse"]), rel=1e-14, abs=1e-15)


# ------------------------------------------------------------ paged caches
def test_gather_paged_hand_example():
    """A hand-laid pool: two sequences (3 and 2 tokens), pages of 2 rows.
    Sequence 0 uses pages 2 then 0, sequence 1 uses page 1; row values name
    their (page, row)."""
    pages = np.array([[[0], [1]], [[10], [11]], [[20], [21]]], dtype=np.uint16)  # [page, row, width 1]
    table = np.array([[2, 0], [1, 1]], dtype=np.int32)
    cu = np.array([0, 3, 5], dtype=np.int32)
    got = oracle.gather_paged(pages, table, cu, 2)
    assert got[:, 0].tolist() == [20, 21, 0, 10, 11]


def test_gather_paged_inverts_the_pool_layout():
    """The oracle's gather undoes the shuffled page pool built by the input
    generator (an independent scatter), for several page sizes."""
    x = workloads.make_inputs(workloads.WORKLOADS[1])
    for ps in (16, 32, 64):
        p = workloads.make_paged(x, ps, seed=ps)
        k = oracle.gather_paged(p.k_pages.view(torch.int16).numpy().view(np.uint16), p.block_table.numpy(),
                                x.cu_seqlens.numpy(), ps)
        assert np.array_equal(k, x.bits("k")), ps


def test_paged_decode_equals_packed_decode():
    """Attention over the paged layout is the attention over the same rows
    packed (the layout changes where rows live, not what is computed)."""
    spec = workloads.with_shape(workloads.WORKLOADS[1], lens=(17, 0, 33, 64))
    x = workloads.make_inputs(spec)
    p = workloads.make_paged(x, 16, seed=3)
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    o1, l1 = oracle.gqa_decode(x.bits("q"), x.bits("k"), x.bits("v"), x.cu_seqlens.numpy(), 2, spec.scale,
                               oracle.F16)
    o2, l2 = oracle.gqa_decode_paged(x.bits("q"), u16(p.k_pages), u16(p.v_pages), p.block_table.numpy(),
                                     x.cu_seqlens.numpy(), 2, spec.scale, oracle.F16)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------ several new query tokens
def whole_prompt_reference(qfull, k, v, num_kv_heads, scale):
    """Causal self-attention of a whole prompt (every position is a query):
    torch's scaled_dot_product_attention(is_causal=True) in float64, key/value
    heads repeated to the query heads.  Returns (out [L, Hq, D], lse [L, Hq])."""
    L, Hq, D = qfull.shape
    G = Hq // num_kv_heads
    qd = qfull.to(torch.float64).permute(1, 0, 2)                               # [Hq, L, D]
    kd = k.to(torch.float64).permute(1, 0, 2).repeat_interleave(G, dim=0)
    vd = v.to(torch.float64).permute(1, 0, 2).repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=True, scale=scale)
    scores = (qd @ kd.transpose(1, 2)) * scale
    scores = scores.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), -math.inf)
    return o.permute(1, 0, 2).numpy(), torch.logsumexp(scores, dim=-1).permute(1, 0).numpy()


def run_varlen(q, k, v, cu_q, cu_k, num_kv_heads, scale, dtype, causal=True):
    dt = oracle.F16 if dtype == torch.float16 else oracle.BF16
    return oracle.gqa_varlen(bits(q), bits(k), bits(v), np.asarray(cu_q, dtype=np.int32),
                             np.asarray(cu_k, dtype=np.int32), num_kv_heads, scale, dt, causal=causal)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 1), (3, 3)])
def test_varlen_whole_prompt_equals_causal_sdpa(Hq, Hkv):
    """Every token of the prompt is new (Lq = Lk): plain causal self-attention."""
    gen = torch.Generator().manual_seed(300 + Hq)
    lens = [1, 7, 40]
    cu = workloads.cu_from_lens(lens)
    T, D = int(cu[-1]), 32
    q = rand16((T, Hq, D), torch.float16, gen)
    k = rand16((T, Hkv, D), torch.float16, gen)
    v = rand16((T, Hkv, D), torch.float16, gen)
    out, lse = run_varlen(q, k, v, cu, cu, Hkv, 0.3, torch.float16)
    for b in range(len(lens)):
        s, e = int(cu[b]), int(cu[b + 1])
        ro, rl = whole_prompt_reference(q[s:e], k[s:e], v[s:e], Hkv, 0.3)
        np.testing.assert_allclose(out[s:e], ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[s:e], rl, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("Lq", [1, 3, 16])
def test_varlen_chunk_equals_tail_of_whole_prompt(Lq):
    """Chunked prefill: the last Lq tokens of a prompt, attended against the
    whole cache, give the same rows as attending the whole prompt at once
    (the new tokens sit at the end of the cache)."""
    gen = torch.Generator().manual_seed(400 + Lq)
    Hq, Hkv, D = 4, 2, 24
    lens_k = [Lq, 40, 100]
    prompts = [(rand16((L, Hq, D), torch.bfloat16, gen), rand16((L, Hkv, D), torch.bfloat16, gen),
                rand16((L, Hkv, D), torch.bfloat16, gen)) for L in lens_k]
    q = torch.cat([p[0][-Lq:] for p in prompts])
    k = torch.cat([p[1] for p in prompts])
    v = torch.cat([p[2] for p in prompts])
    cu_q = workloads.cu_from_lens([Lq] * len(lens_k))
    cu_k = workloads.cu_from_lens(lens_k)
    out, lse = run_varlen(q, k, v, cu_q, cu_k, Hkv, 0.25, torch.bfloat16)
    for b, (qf, kf, vf) in enumerate(prompts):
        ro, rl = whole_prompt_reference(qf, kf, vf, Hkv, 0.25)
        np.testing.assert_allclose(out[b * Lq:(b + 1) * Lq], ro[-Lq:], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b * Lq:(b + 1) * Lq], rl[-Lq:], rtol=1e-13, atol=1e-13)


def test_varlen_without_mask_equals_sdpa():
    gen = torch.Generator().manual_seed(500)
    Hq, Hkv, D, Lq, Lk = 6, 3, 16, 5, 29
    q = rand16((Lq, Hq, D), torch.float16, gen)
    k = rand16((Lk, Hkv, D), torch.float16, gen)
    v = rand16((Lk, Hkv, D), torch.float16, gen)
    out, lse = run_varlen(q, k, v, [0, Lq], [0, Lk], Hkv, 0.2, torch.float16, causal=False)
    qd = q.to(torch.float64).permute(1, 0, 2)
    kd = k.to(torch.float64).permute(1, 0, 2).repeat_interleave(2, dim=0)
    vd = v.to(torch.float64).permute(1, 0, 2).repeat_interleave(2, dim=0)
    ro = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, scale=0.2).permute(1, 0, 2).numpy()
    rl = torch.logsumexp((qd @ kd.transpose(1, 2)) * 0.2, dim=-1).permute(1, 0).numpy()
    np.testing.assert_allclose(out, ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_varlen_rows_that_see_no_key():
    """More new tokens than cached rows: the first Lq - Lk new tokens see no
    key (out 0, lse -inf); the others see keys 0 .. i - (Lq - Lk).  An empty
    query range contributes no rows."""
    gen = torch.Generator().manual_seed(600)
    Hq, D, Lq, Lk = 2, 8, 5, 3
    q = rand16((Lq, Hq, D), torch.float16, gen)
    k = rand16((Lk, 1, D), torch.float16, gen)
    v = rand16((Lk, 1, D), torch.float16, gen)
    kk = torch.cat([rand16((4, 1, D), torch.float16, gen), k])
    vv = torch.cat([rand16((4, 1, D), torch.float16, gen), v])
    out, lse = run_varlen(q, kk, vv, [0, 0, Lq], [0, 4, 4 + Lk], 1, 1.0, torch.float16)
    assert np.all(out[:Lq - Lk] == 0) and np.all(lse[:Lq - Lk] == -np.inf)
    ro, rl = whole_prompt_reference(q[Lq - Lk:], k, v, 1, 1.0)
    np.testing.assert_allclose(out[Lq - Lk:], ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[Lq - Lk:], rl, rtol=1e-13, atol=1e-13)


def test_mla_varlen_equals_gqa_varlen_with_materialised_value():
    gen = torch.Generator().manual_seed(700)
    lens_q, lens_k = [2, 1, 4], [9, 1, 40]
    cu_q, cu_k = workloads.cu_from_lens(lens_q), workloads.cu_from_lens(lens_k)
    H, R, P = 4, 32, 8
    q = rand16((int(cu_q[-1]), H, R + P), torch.bfloat16, gen)
    c = rand16((int(cu_k[-1]), R + P), torch.bfloat16, gen)
    out, lse = oracle.mla_varlen(bits(q), bits(c), cu_q.numpy(), cu_k.numpy(), 0.17, oracle.BF16,
                                 kv_lora_rank=R, rope_dim=P)
    vcopy = c[:, :R].contiguous()
    ro, rl = oracle.varlen_attn(bits(q), bits(c), bits(vcopy), cu_q.numpy(), cu_k.numpy(), 1, R + P, R,
                                R + P, R, 0.17, oracle.BF16)
    np.testing.assert_array_equal(out, ro)
    np.testing.assert_array_equal(lse, rl)
