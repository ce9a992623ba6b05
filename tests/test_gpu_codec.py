"""GPU parity of the INT8 all-reduce payload codec: the HIP kernels (through
the C ABI) against the oracle (oracle/codec.py) on identical seeded payloads.
Codes, scales and 16-bit values are integers or bit patterns decided in the
same fp32 steps on both sides, so they must match exactly.  A simulated ring
all-reduce over eight payloads on one GPU checks the hop kernel in its use,
against the oracle's hops (exactly) and against the fp64 sum (within the
coding error the hops accumulate)."""
import numpy as np
import pytest
import torch

from oracle import codec

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


def code_of(dt):
    return codec.F16 if dt == torch.float16 else codec.BF16


def payload(n, dt, seed, zero_chunk=None):
    """Seeded N(0,1) values with magnitudes that differ by up to 2^12 between
    runs of 64 elements (rounded once to dt); optionally one all-zero span."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, generator=g)
    x = x * torch.exp2(torch.randint(-6, 6, (n // 64 + 1,), generator=g).float()).repeat_interleave(64)[:n]
    if zero_chunk is not None:
        x[zero_chunk[0]:zero_chunk[1]] = 0
    return x.to(dt)


def bits(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


CASES = [(n, chunk, dt) for n, chunk in [(1, 512), (255, 256), (256, 256), (1000, 512), (65573, 1024),
                                         (1 << 20, 512), (3 * 1024 * 1024 + 5, 256)]
         for dt in (torch.float16, torch.bfloat16)]


@pytest.mark.parametrize("n,chunk,dt", CASES)
def test_quantize_dequantize_bit_exact(n, chunk, dt):
    x = payload(n, dt, n % 997 + chunk, zero_chunk=(chunk, 2 * chunk) if n > 2 * chunk else None)
    codes, scales = zl().zl_int8_quantize(x.to(DEV), chunk=chunk)
    back = zl().zl_int8_dequantize(codes, scales, dtype=dt, chunk=chunk)
    torch.cuda.synchronize()
    rc, rs = codec.quantize(bits(x), code_of(dt), chunk)
    assert np.array_equal(codes.cpu().numpy(), rc), "codes"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32)), "scales"
    assert np.array_equal(bits(back), codec.dequantize(rc, rs, chunk, code_of(dt))), "dequantized values"


@pytest.mark.parametrize("chunk,dt", [(256, torch.float16), (512, torch.bfloat16), (1024, torch.float16)])
@pytest.mark.parametrize("outputs", ["both", "codes", "sum"])
def test_reduce_step_bit_exact(chunk, dt, outputs):
    n = 200_003
    a = payload(n, dt, 1)
    local = payload(n, dt, 2)
    rc, rs = codec.quantize(bits(a), code_of(dt), chunk)
    co, so, su = zl().zl_int8_reduce_step(torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV),
                                          local.to(DEV), chunk=chunk, code_out=outputs != "sum",
                                          write_sum=outputs != "codes")
    torch.cuda.synchronize()
    oc, os_, osum = codec.reduce_step(rc, rs, bits(local), code_of(dt), chunk)
    if outputs != "sum":
        assert np.array_equal(co.cpu().numpy(), oc)
        assert np.array_equal(so.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    else:
        assert co is None and so is None
    if outputs != "codes":
        assert np.array_equal(bits(su), osum)
    else:
        assert su is None


def test_ring_all_reduce_of_eight_payloads():
    """Reduce-scatter then all-gather over eight payloads, with every hop's
    data coded: hop kernels against the oracle's hops (exact), the result
    against the fp64 sum (within the accumulated coding error)."""
    R, seg, chunk, dt = 8, 64 * 1024, 512, torch.float16
    xs = [payload(R * seg, dt, 100 + r) for r in range(R)]
    dev_x = [x.to(DEV) for x in xs]
    sl = lambda k: slice(k * seg, (k + 1) * seg)
    # reduce-scatter: at step t, rank r sends its running partial of segment
    # (r - t) mod R to rank r+1, which adds its own values and codes it again
    gpu = {r: zl().zl_int8_quantize(dev_x[r][sl(r % R)].contiguous(), chunk=chunk) for r in range(R)}
    ref = {r: codec.quantize(bits(xs[r][sl(r % R)]), codec.F16, chunk) for r in range(R)}
    for t in range(1, R):
        new_gpu, new_ref = {}, {}
        for r in range(R):
            dst, k = (r + 1) % R, (r - t + 1) % R
            local = dev_x[dst][sl(k)].contiguous()
            last = t == R - 1
            c, s, su = zl().zl_int8_reduce_step(gpu[r][0], gpu[r][1], local, chunk=chunk, write_sum=last)
            oc, os_, osum = codec.reduce_step(ref[r][0], ref[r][1], bits(xs[dst][sl(k)]), codec.F16, chunk)
            new_gpu[dst], new_ref[dst] = (c, s, su), (oc, os_, osum)
        gpu, ref = new_gpu, new_ref
    torch.cuda.synchronize()
    for r in range(R):
        assert np.array_equal(gpu[r][0].cpu().numpy(), ref[r][0])
        assert np.array_equal(bits(gpu[r][2]), ref[r][2])
    # all-gather of the coded, fully reduced segments; every rank decodes them
    full = torch.empty(R * seg, dtype=dt, device=DEV)
    for r in range(R):
        k = (r + 1) % R  # the segment rank r holds after the reduce-scatter
        full[sl(k)] = zl().zl_int8_dequantize(gpu[r][0], gpu[r][1], dtype=dt, chunk=chunk)
    torch.cuda.synchronize()
    exact = np.sum([x.double().numpy() for x in xs], axis=0)
    got = full.double().cpu().numpy()
    # each of the R-1 hops codes its partial once (error <= scale/2 of that
    # partial), the all-gather codes the total once more, plus fp16 rounding
    amax = np.max(np.abs(np.sum([np.abs(x.double().numpy()) for x in xs], axis=0)).reshape(-1, chunk), axis=1)
    bound = np.repeat(amax / 127 * 0.5 * R + amax * 2.0 ** -10, chunk)
    assert np.all(np.abs(got - exact) <= bound)
