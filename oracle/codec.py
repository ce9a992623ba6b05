"""Plain CPU oracle of the INT8 all-reduce payload codec.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The GPU library never imports it
and shares no code with it.

What is computed.  ZhiLight quantises the payload of its tensor-parallel
all-reduce from 16-bit floats to 8-bit integers to cut the bytes that cross
between GPUs (first page, section 1 on dual streams and the INT8 all-reduce;
second page, section "Dual streams, host all-reduce and the memory model";
the talk notes' section on all-reduce data quantisation).  The pages give no
scheme; the reading here is the plain one: the payload is cut into chunks of
`chunk` consecutive elements, each chunk carries one fp32 scale, and every
element is coded symmetrically with 127 levels per sign:

    amax  = max |x| over the chunk
    r     = 127 / amax              (0 when amax = 0)
    code  = rint(x * r)             (round half to even), in [-127, 127]
    scale = amax / 127
    x'    = code * scale

One hop of a ring all-reduce on one GPU receives a coded chunk, adds its own
16-bit values and codes the sum again for the next hop (and writes the sum
in 16 bits on the last hops):

    y = code_in * scale_in + local

A code is an integer decided by floating point, so these steps are taken in
fp32, the precision of the GPU kernels, with every product and sum rounded on
its own (no fused multiply-add); numpy float32 arithmetic is IEEE
round-to-nearest-even, and fp16/bf16 inputs are exactly representable in
fp32.  A last chunk shorter than `chunk` is coded on its own.
"""
import numpy as np
import torch

F16 = 0
BF16 = 1


def to_f32(bits, dtype: int) -> np.ndarray:
    """Exact fp32 values of 16-bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float32)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to16(x32: np.ndarray, dtype: int) -> np.ndarray:
    """fp32 -> 16-bit patterns, round to nearest even."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)
    return torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_f32(x32: np.ndarray, chunk: int):
    """Per-chunk codes (int8) and scales (fp32) of fp32 values."""
    x32 = np.asarray(x32, dtype=np.float32)
    n = x32.size
    nchunks = (n + chunk - 1) // chunk
    codes = np.zeros(n, dtype=np.int8)
    scales = np.zeros(nchunks, dtype=np.float32)
    for c in range(nchunks):
        seg = x32[c * chunk:(c + 1) * chunk]
        amax = np.float32(np.max(np.abs(seg)))
        if amax == 0:
            continue
        r = np.float32(127) / amax
        q = np.rint(seg * r)
        codes[c * chunk:(c + 1) * chunk] = np.clip(q, -127, 127).astype(np.int8)
        scales[c] = amax / np.float32(127)
    return codes, scales


def quantize(bits, dtype: int, chunk: int):
    """Codes and scales of a 16-bit payload (raw patterns)."""
    return quantize_f32(to_f32(bits, dtype), chunk)


def dequantize_f32(codes, scales, chunk: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int8)
    s = np.repeat(np.asarray(scales, dtype=np.float32), chunk)[:codes.size]
    return codes.astype(np.float32) * s


def dequantize(codes, scales, chunk: int, dtype: int) -> np.ndarray:
    """16-bit patterns of code * scale."""
    return to16(dequantize_f32(codes, scales, chunk), dtype)


def reduce_step(codes_in, scales_in, local_bits, dtype: int, chunk: int):
    """One ring hop: y = code_in * scale_in + local, in fp32.  Returns
    (codes_out, scales_out, sum16) with sum16 the 16-bit patterns of y."""
    y = dequantize_f32(codes_in, scales_in, chunk) + to_f32(local_bits, dtype)
    codes, scales = quantize_f32(y, chunk)
    return codes, scales, to16(y, dtype)
