"""Decode calls captured in a HIP graph (torch.cuda.graph) and replayed: the
library enqueues kernels only (no allocation, no memset, no host sync), so a
captured call is replayable.  Each replay, with eager calls and
synchronisations between replays, must give bitwise the eager result, also
after the captured inputs are overwritten in place."""
import math

import numpy as np
import pytest
import torch

import workloads
from tests.parity import gate
from tests.test_gpu_parity import DEV, run_oracle

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


@pytest.mark.parametrize("kind", ["gqa", "mla"])
def test_captured_decode_replays_bitwise(kind):
    if kind == "mla":
        spec = workloads.Spec("graph-mla", "mla", 6, 16, 1, 576, 512, (700, 33, 2100, 0, 257, 64), "bf16",
                              float(np.float32(1 / math.sqrt(192))), 21)
    else:
        spec = workloads.Spec("graph-gqa", "gqa", 6, 8, 2, 128, 128, (700, 33, 2100, 0, 257, 64), "f16",
                              float(np.float32(1 / math.sqrt(128))), 22)
    x = workloads.make_inputs(spec)
    x2 = workloads.make_inputs(spec, seed=spec.seed + 100)   # same shapes, other values
    q, cu = x.q.to(DEV), x.cu_seqlens.to(DEV)
    if kind == "mla":
        kv = (x.latent.to(DEV),)
        ws = zl().new_workspace(zl().zl_decode_attn_mla_workspace_size(spec.batch, spec.num_q_heads, 512, 64,
                                                                      x.max_seqlen, spec.torch_dtype), DEV)
    else:
        kv = (x.k.to(DEV), x.v.to(DEV))
        ws = zl().new_workspace(zl().zl_decode_attn_workspace_size(spec.batch, spec.num_q_heads, spec.num_kv_heads,
                                                                  128, x.max_seqlen, spec.torch_dtype), DEV)
    out = torch.empty(spec.batch, spec.num_q_heads, spec.head_dim_v, dtype=spec.torch_dtype, device=DEV)
    lse = torch.empty(spec.batch, spec.num_q_heads, dtype=torch.float32, device=DEV)

    def call(stream=None):
        if kind == "mla":
            zl().zl_decode_attn_mla(q, kv[0], cu, x.max_seqlen, spec.scale, out=out, lse=lse, workspace=ws,
                                    stream=stream)
        else:
            zl().zl_decode_attn_gqa(q, kv[0], kv[1], cu, x.max_seqlen, spec.scale, out=out, lse=lse, workspace=ws,
                                    stream=stream)

    call()
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()
    ro, rl = run_oracle(x)
    gate(eager_out, ro, spec.torch_dtype, eager_lse, rl, where=f"{kind} eager")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(stream=s)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(stream=torch.cuda.current_stream())
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("inf"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out) and torch.equal(lse, eager_lse), f"{kind} replay {i}"
        call()   # an eager call between replays, on the same buffers
        torch.cuda.synchronize()
    # new values in the captured input buffers: the replay reads them
    q.copy_(x2.q.to(DEV))
    for t, src in zip(kv, (x2.latent,) if kind == "mla" else (x2.k, x2.v)):
        t.copy_(src.to(DEV))
    out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    ro2, rl2 = run_oracle(x2)
    gate(out, ro2, spec.torch_dtype, lse, rl2, where=f"{kind} replay on new inputs")
