"""Pins of the INT8 payload codec oracle (oracle/codec.py) against things
other than itself: hand-derived examples (tests/golden/int8_codec_examples.txt),
the rounding error bound of symmetric 127-level coding, and invariants of the
scheme (the largest element codes to +-127, power-of-two scaling moves only the
scale, a short last chunk is coded on its own, adding a zero payload codes the
local values).  tests/test_oracle_codec.py::test_codec_mutants_are_caught
plants plausible slips and checks that these pins catch each."""
import os
import re
import types

import numpy as np
import pytest
import torch

from oracle import codec

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "int8_codec_examples.txt")
DT = {"f16": codec.F16, "bf16": codec.BF16}


def bits16(vals, dtype):
    t = torch.tensor(vals, dtype=torch.float32).to(torch.float16 if dtype == codec.F16 else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def fp32_quot(expr):
    a, b = expr.split("/")
    return np.float32(np.float32(float(a)) / np.float32(float(b))) if float(b) else np.float32(0)


def golden_cases():
    text = open(GOLDEN).read()
    cases = []
    for head, body in re.findall(r"\[(\w+ \w+)\]\n((?:[^\[\n#][^\n]*\n?)+)", text):
        kv = dict(line.split(" = ", 1) for line in body.strip().splitlines())
        cases.append((head, kv))
    return cases


def test_golden_examples(mod=codec):
    cases = golden_cases()
    assert len(cases) == 6
    for head, kv in cases:
        dt, chunk = DT[kv["dtype"]], int(kv["chunk"])
        want_codes = np.array(kv["codes"].split(), dtype=np.int8)
        want_scales = np.array([fp32_quot(e) for e in kv["scales"].split()], dtype=np.float32)
        if head.startswith("quantize"):
            codes, scales = mod.quantize(bits16([float(v) for v in kv["x"].split()], dt), dt, chunk)
        else:
            codes, scales, s16 = mod.reduce_step(np.array(kv["codes_in"].split(), dtype=np.int8),
                                                 np.array(kv["scales_in"].split(), dtype=np.float32),
                                                 bits16([float(v) for v in kv["local"].split()], dt), dt, chunk)
            assert np.array_equal(s16, bits16([float(v) for v in kv["sum"].split()], dt)), head
        assert np.array_equal(codes, want_codes), (head, codes)
        assert np.array_equal(scales, want_scales), (head, scales)


def random_payload(n, dtype, seed, spread=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, generator=g)
    if spread:  # chunks of very different magnitudes
        x = x * torch.exp2(torch.randint(-12, 12, (n // 64 + 1,), generator=g).float()).repeat_interleave(64)[:n]
    t = x.to(torch.float16 if dtype == codec.F16 else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", [codec.F16, codec.BF16])
@pytest.mark.parametrize("chunk", [64, 256, 1024])
def test_round_trip_error_bound(dtype, chunk, mod=codec):
    """|x - code*scale| <= scale/2 plus fp32 rounding (amax * 2^-20)."""
    b = random_payload(5000, dtype, chunk + dtype)
    x = codec.to_f32(b, dtype).astype(np.float64)
    codes, scales = mod.quantize(b, dtype, chunk)
    xr = mod.dequantize_f32(codes, scales, chunk).astype(np.float64)
    s = np.repeat(scales.astype(np.float64), chunk)[:x.size]
    amax = s * 127
    assert np.all(np.abs(xr - x) <= s / 2 + amax * 2.0 ** -20)


@pytest.mark.parametrize("dtype", [codec.F16, codec.BF16])
def test_largest_element_codes_to_127(dtype, mod=codec):
    b = random_payload(4096, dtype, 11)
    x = codec.to_f32(b, dtype)
    codes, scales = mod.quantize(b, dtype, 256)
    assert codes.min() >= -127 and codes.max() <= 127
    for c in range(16):
        seg = x[c * 256:(c + 1) * 256]
        i = int(np.argmax(np.abs(seg)))
        assert codes[c * 256 + i] == (127 if seg[i] > 0 else -127)
        assert scales[c] == np.float32(np.abs(seg).max()) / np.float32(127)


def test_power_of_two_scaling_moves_only_the_scale(mod=codec):
    b = random_payload(2048, codec.F16, 5, spread=False)
    x = codec.to_f32(b, codec.F16)
    c1, s1 = mod.quantize_f32(x, 512)
    c2, s2 = mod.quantize_f32(x * np.float32(8), 512)
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * np.float32(8))


def test_zero_chunk_and_short_tail(mod=codec):
    b = random_payload(1000, codec.BF16, 7)
    b[256:512] = 0
    codes, scales = mod.quantize(b, codec.BF16, 256)
    assert np.all(codes[256:512] == 0) and scales[1] == 0
    tc, ts = mod.quantize(b[768:], codec.BF16, 256)
    assert np.array_equal(codes[768:], tc) and scales[3] == ts[0]


def test_reduce_step_with_zero_payload_codes_the_local_values(mod=codec):
    b = random_payload(1500, codec.F16, 9)
    codes, scales, s16 = mod.reduce_step(np.zeros(1500, np.int8), np.zeros(3, np.float32), b, codec.F16, 512)
    qc, qs = mod.quantize(b, codec.F16, 512)
    assert np.array_equal(codes, qc) and np.array_equal(scales, qs) and np.array_equal(s16, b)


MUTANTS = {
    "truncate-not-round": ("q = np.rint(seg * r)", "q = np.trunc(seg * r)"),
    "128-levels": ("r = np.float32(127) / amax", "r = np.float32(128) / amax"),
    "scale-not-divided": ("scales[c] = amax / np.float32(127)", "scales[c] = amax"),
    "absmax-without-abs": ("amax = np.float32(np.max(np.abs(seg)))", "amax = np.float32(np.max(seg))"),
    "reduce-drops-local": ("y = dequantize_f32(codes_in, scales_in, chunk) + to_f32(local_bits, dtype)",
                           "y = dequantize_f32(codes_in, scales_in, chunk)"),
    "scale-of-next-chunk": ("s = np.repeat(np.asarray(scales, dtype=np.float32), chunk)[:codes.size]",
                            "s = np.repeat(np.roll(np.asarray(scales, dtype=np.float32), 1), chunk)[:codes.size]"),
}


def _battery(mod):
    return [lambda: test_golden_examples(mod),
            lambda: test_round_trip_error_bound(codec.F16, 256, mod),
            lambda: test_largest_element_codes_to_127(codec.BF16, mod),
            lambda: test_power_of_two_scaling_moves_only_the_scale(mod),
            lambda: test_zero_chunk_and_short_tail(mod),
            lambda: test_reduce_step_with_zero_payload_codes_the_local_values(mod)]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_codec_mutants_are_caught(name):
    src = open(codec.__file__).read()
    old, new = MUTANTS[name]
    assert old in src, name
    mod = types.ModuleType(f"codec_{name}")
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = 0
    for pin in _battery(mod):
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught, f"no pin caught mutant {name}"
