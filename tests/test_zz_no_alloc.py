"""GPU check of zl_decode_attn_gqa_no_alloc (through the C ABI): on two calls
in a row, the second with a smaller batch, it gives the bits of
zl_decode_attn_gqa (same kernels, same split) and passes the parity gate
against the oracle.  Outputs are guarded (NaN / +inf pre-fill, canaries)."""
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


def one_call(x, where):
    import mla_attention_amd as zl
    s = x.spec
    q, k, v, cu = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), x.cu_seqlens.to(DEV)
    bufs = CallBuffers(s.batch, s.num_q_heads, s.head_dim_v, s.torch_dtype, DEV)
    out, lse = zl.zl_decode_attn_gqa_no_alloc(q, k, v, cu, x.max_seqlen, s.scale, out=bufs.out.t, lse=bufs.lse.t)
    torch.cuda.synchronize()
    bufs.check(where)
    ref_out, ref_lse = zl.zl_decode_attn_gqa(q, k, v, cu, x.max_seqlen, s.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), where
    dt = oracle.F16 if s.dtype == "f16" else oracle.BF16
    ro, rl = oracle.gqa_decode(x.bits("q"), x.bits("k"), x.bits("v"), x.cu_seqlens.numpy(), s.num_kv_heads, s.scale,
                               dt)
    gate(out, ro, s.torch_dtype, lse, rl, where=where)


def test_no_alloc_matches_the_workspace_call_on_two_calls_in_a_row():
    big = workloads.make_inputs(workloads.WORKLOADS[2])
    one_call(big, "no-alloc, first call: llama3-8b-decode-b32-h32kv8-d128")
    small_spec = workloads.with_shape(workloads.WORKLOADS[1], batch=3, lens=(5, 130, 0), dtype="bf16")
    small = workloads.make_inputs(small_spec, seed=17)
    one_call(small, "no-alloc, second call: 3 sequences, D 64, bf16")


def test_no_alloc_head_dims_and_empty_batch():
    import mla_attention_amd as zl
    spec = workloads.with_shape(workloads.WORKLOADS[3], batch=5, lens=(1, 4000, 33, 0, 700))
    one_call(workloads.make_inputs(spec, seed=18), "no-alloc, 8/1 heads, D 128")
    # batch 0 is a no-op
    e = torch.empty(0, 8, 128, dtype=torch.float16, device=DEV)
    kv = torch.empty(0, 1, 128, dtype=torch.float16, device=DEV)
    zl.zl_decode_attn_gqa_no_alloc(e, kv, kv, torch.zeros(1, dtype=torch.int32, device=DEV), 0, 0.1)
    torch.cuda.synchronize()
