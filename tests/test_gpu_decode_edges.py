"""Decode edge cases on the GPU: the closed forms and invariances that pin the
oracle (uniform weights, a negative scale, a large constant added to every
score, duplicated rows) run through the decode kernels, GQA and MLA, packed
and paged, both 16-bit types.  Each case is checked against the oracle on the
same bits and, where the attention has a closed form, against that form too.
Outputs are guarded (NaN / +inf pre-fill, canaries) as in test_gpu_parity.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from tests.parity import LSE_ABS, LSE_REL, gate
from tests.test_gpu_parity import run_gpu, run_gpu_paged, run_oracle, run_oracle_paged

pytestmark = pytest.mark.gpu

LENS = (1, 33, 700, 2100, 64, 0, 257)  # one empty sequence, ragged tails, split sequences
SHIFT = 50.0                            # |scale * q . u| of the key shift


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_amd as zl
    zl.library()
    yield


def base_inputs(kind, dt, lens=LENS):
    d = "f16" if dt == torch.float16 else "bf16"
    if kind == "mla":
        spec = workloads.Spec("edge-mla", "mla", len(lens), 16, 1, 576, 512, tuple(lens), d,
                              float(np.float32(1 / math.sqrt(192))), 13)
    else:
        spec = workloads.Spec("edge-gqa", "gqa", len(lens), 8, 2, 128, 128, tuple(lens), d,
                              float(np.float32(1 / math.sqrt(128))), 12)
    return workloads.make_inputs(spec)


def with_scale(x, scale):
    x.spec = workloads.with_shape(x.spec, scale=float(np.float32(scale)))
    return x


def key_shift(x):
    """K' = K + 1 u^T for every row of a sequence (u per sequence and key head),
    with scale * q . u = SHIFT for the first query head of each group.  MLA
    shifts only the 64 rotary columns, which the value does not include."""
    s = x.spec
    cu = x.cu_seqlens.numpy()
    for b in range(s.batch):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 == r0:
            continue
        if s.kind == "mla":
            qr = x.q[b, 0, 512:].double()
            u = SHIFT / s.scale * qr / qr.dot(qr)
            x.latent[r0:r1, 512:] = (x.latent[r0:r1, 512:].double() + u).to(s.torch_dtype)
        else:
            for g in range(s.num_kv_heads):
                qh = x.q[b, g * s.group].double()
                u = SHIFT / s.scale * qh / qh.dot(qh)
                x.k[r0:r1, g] = (x.k[r0:r1, g].double() + u).to(s.torch_dtype)
    return x


def duplicated(x):
    """Every sequence's rows twice over (the sequence then has 2L rows)."""
    s = x.spec
    cu = x.cu_seqlens.numpy()
    lens = [2 * int(v) for v in x.lens]
    spec = workloads.with_shape(s, lens=tuple(lens))
    cu2 = workloads.cu_from_lens(lens)

    def dup(t):
        return torch.cat([torch.cat([t[int(cu[b]):int(cu[b + 1])]] * 2) for b in range(s.batch)])

    if s.kind == "mla":
        return workloads.Inputs(spec, np.asarray(lens), cu2, x.q, latent=dup(x.latent))
    return workloads.Inputs(spec, np.asarray(lens), cu2, x.q, k=dup(x.k), v=dup(x.v))


def values(x):
    """V rows decoded to float64, [T, Hkv, Dv] (MLA: the latent's first 512 columns)."""
    if x.spec.kind == "mla":
        return x.latent[:, :512].double().unsqueeze(1).numpy()
    return x.v.double().numpy()


def mean_of_values(x):
    """The closed form of uniform weights: out[b, h] = mean of sequence b's V
    rows of h's key head, lse = ln L; an empty sequence gives 0 and -inf."""
    s = x.spec
    cu = x.cu_seqlens.numpy()
    v = values(x)
    out = np.zeros((s.batch, s.num_q_heads, s.head_dim_v))
    lse = np.full((s.batch, s.num_q_heads), -np.inf)
    for b in range(s.batch):
        L = int(cu[b + 1] - cu[b])
        if L == 0:
            continue
        for h in range(s.num_q_heads):
            out[b, h] = v[int(cu[b]):int(cu[b + 1]), h // s.group].mean(axis=0)
            lse[b, h] = math.log(L)
    return out, lse


def run(x, paged, where):
    if paged:
        p = workloads.make_paged(x, 16 if x.spec.kind == "gqa" else 64, seed=3)
        out, lse = run_gpu_paged(x, p, where=where)
        ro, rl = run_oracle_paged(x, p)
    else:
        out, lse = run_gpu(x, where=where)
        ro, rl = run_oracle(x)
    gate(out, ro, x.spec.torch_dtype, lse, rl, where=where)
    return out, lse


PARAMS = [(k, dt, paged) for k in ("gqa", "mla") for dt in (torch.float16, torch.bfloat16) for paged in (False, True)]
IDS = [f"{k}-{'f16' if dt == torch.float16 else 'bf16'}-{'paged' if p else 'packed'}" for k, dt, p in PARAMS]


@pytest.mark.parametrize("kind,dt,paged", PARAMS, ids=IDS)
@pytest.mark.parametrize("how", ["scale0", "q0"])
def test_uniform_weights_give_the_mean_of_v(kind, dt, paged, how):
    x = base_inputs(kind, dt)
    if how == "scale0":
        with_scale(x, 0.0)
    else:
        x.q.zero_()
    where = f"{how} {kind} {dt} {'paged' if paged else 'packed'}"
    print(where, flush=True)
    out, lse = run(x, paged, where)
    mo, ml = mean_of_values(x)
    gate(out, mo, dt, lse, ml, where=where + " (closed form)")


@pytest.mark.parametrize("kind,dt,paged", PARAMS, ids=IDS)
def test_negative_scale(kind, dt, paged):
    x = base_inputs(kind, dt)
    with_scale(x, -x.spec.scale)
    where = f"negative scale {kind} {dt} {'paged' if paged else 'packed'}"
    print(where, flush=True)
    run(x, paged, where)


@pytest.mark.parametrize("kind,dt,paged", PARAMS, ids=IDS)
def test_constant_key_shift(kind, dt, paged):
    """A key shift adds a constant (about SHIFT for the first head of each
    group) to every score of a sequence: the kernel's max subtraction must
    absorb it, and lse moves by it."""
    x0 = base_inputs(kind, dt)
    x = key_shift(base_inputs(kind, dt))
    where = f"key shift {kind} {dt} {'paged' if paged else 'packed'}"
    print(where, flush=True)
    _, lse = run(x, paged, where)
    _, l0 = run_oracle(x0)
    s = x.spec
    heads = [g * s.group for g in range(s.num_kv_heads)]
    nonempty = np.asarray(x.lens) > 0
    moved = lse.cpu().numpy()[nonempty][:, heads] - l0[nonempty][:, heads]
    assert np.all(np.abs(moved - SHIFT) < 0.5), moved


@pytest.mark.parametrize("kind,dt,paged", PARAMS, ids=IDS)
def test_duplicated_rows_add_ln2(kind, dt, paged):
    x0 = base_inputs(kind, dt)
    x = duplicated(x0)
    where = f"duplicated rows {kind} {dt} {'paged' if paged else 'packed'}"
    print(where, flush=True)
    out, lse = run(x, paged, where)
    ro, rl = run_oracle(x0)
    fin = np.isfinite(rl)
    gate(out, ro, dt, where=where + " (against the undoubled rows)")
    shifted = lse.cpu().numpy().astype(np.float64)[fin] - math.log(2.0)
    assert np.all(np.abs(shifted - rl[fin]) <= LSE_ABS + LSE_REL * np.abs(rl[fin])), where
    assert np.all(np.isneginf(lse.cpu().numpy()[~fin]))


def permuted(x, seed=7):
    """Every sequence's rows in a seeded random order (the same order for K
    and V, or for the latent rows): the attention does not depend on it."""
    s = x.spec
    cu = x.cu_seqlens.numpy()
    rng = np.random.default_rng(seed)
    order = np.concatenate([int(cu[b]) + rng.permutation(int(cu[b + 1] - cu[b])) for b in range(s.batch)])
    idx = torch.from_numpy(order.astype(np.int64))
    if s.kind == "mla":
        return workloads.Inputs(s, np.asarray(x.lens), x.cu_seqlens, x.q, latent=x.latent[idx].contiguous())
    return workloads.Inputs(s, np.asarray(x.lens), x.cu_seqlens, x.q, k=x.k[idx].contiguous(),
                            v=x.v[idx].contiguous())


@pytest.mark.parametrize("kind,dt,paged", PARAMS, ids=IDS)
def test_token_permutation(kind, dt, paged):
    """Rows of every sequence shuffled: the kernel's result on the shuffled
    caches meets the gate against the oracle on the original order (the
    split points and tile boundaries now fall on other rows)."""
    x0 = base_inputs(kind, dt)
    x = permuted(x0)
    where = f"permuted rows {kind} {dt} {'paged' if paged else 'packed'}"
    print(where, flush=True)
    out, lse = run(x, paged, where)
    ro, rl = run_oracle(x0)
    gate(out, ro, dt, lse, rl, where=where + " (against the original order)")
