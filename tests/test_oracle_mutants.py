"""Plant plausible slips in a copy of the oracle and check the pins catch each.

Every mutant is a one-line textual change to oracle/zl_oracle.c compiled on
the CPU into a temporary library; the pin battery of test_oracle_pins.py is
then run against it and at least one pin must fail.  Every mutation keeps all
memory accesses in bounds.  Nothing here touches a GPU.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import build as obuild

from . import test_oracle_pins as pins

MUTANTS = {
    "drop-scale": ("s[i] = scale * acc;", "s[i] = acc;"),
    "interleaved-head-map": ("int g = h / group;", "int g = h % num_kv_heads;"),
    "no-normalisation": ("out[e] /= l;", "out[e] /= 1.0;"),
    "lse-log2": ("*lse = m + log(l);", "*lse = m + log2(l);"),
    "lse-without-max": ("*lse = m + log(l);", "*lse = log(l);"),
    "weight-sign": ("s[i] = exp(s[i] - m);", "s[i] = exp(m - s[i]);"),
    "v-dims-reversed": ("out[e] += s[i] * dec(vrow[e], dtype);",
                        "out[e] += s[i] * dec(vrow[dv - 1 - e], dtype);"),
    "k-stride-ignored": ("dec(k[(long)i * k_stride + d], dtype)", "dec(k[(long)i * dk + d], dtype)"),
    "last-token-dropped-in-pv": ("for (int i = 0; i < L; ++i) {\n        const uint16_t *vrow",
                                 "for (int i = 0; i < L - 1; ++i) {\n        const uint16_t *vrow"),
    "sequence-base-unscaled": ("k + (long)cu[b] * k_row_stride + (long)g * dk",
                               "k + (long)cu[b] + (long)g * dk"),
    "combine-weight-unshifted": ("double w = exp(part_lse[(long)s * rows + r] - M);",
                                 "double w = exp(part_lse[(long)s * rows + r]);"),
    "combine-lse-without-max": ("lse[r] = M + log(wsum);", "lse[r] = log(wsum);"),
    "f16-bias-off-by-one": ("v = ldexp((double)(m | 0x400), e - 25);", "v = ldexp((double)(m | 0x400), e - 24);"),
    "bf16-hidden-bit-missing": ("v = ldexp((double)(m | 0x80), e - 134);", "v = ldexp((double)m, e - 134);"),
    "f16-subnormal-scale": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "varlen-causal-off-by-one": ("int L = causal ? Lk - Lq + i + 1 : Lk;", "int L = causal ? Lk - Lq + i : Lk;"),
    "varlen-top-left-causal": ("int L = causal ? Lk - Lq + i + 1 : Lk;", "int L = causal ? i + 1 : Lk;"),
    "varlen-query-row-within-sequence": ("attend_one(q + (t * num_q_heads + h) * dk,",
                                         "attend_one(q + ((long)i * num_q_heads + h) * dk,"),
    "mla-value-offset": ("return zo_decode_attn(q, latent, latent, cu,", "return zo_decode_attn(q, latent, latent + rope_dim, cu,"),
}


def _battery():
    """The pins, each bound to fixed arguments, as zero-argument callables."""
    return [
        lambda: pins.test_p11_decoders_all_patterns(torch.float16, oracle.F16),
        lambda: pins.test_p11_decoders_all_patterns(torch.bfloat16, oracle.BF16),
        lambda: pins.test_matches_torch_sdpa_float64(torch.float16, 8, 2, 64),
        lambda: pins.test_matches_torch_sdpa_float64(torch.bfloat16, 16, 1, 72),
        pins.test_config1_matches_torch_sdpa,
        lambda: pins.test_p1_uniform_weights_give_mean_of_v(False),
        pins.test_p2_single_token_returns_its_value,
        pins.test_empty_sequence_gives_zero_and_minus_inf,
        pins.test_p3_constant_added_to_scores,
        pins.test_p4_naive_softmax_long_double_bruteforce,
        pins.test_p6_duplicating_every_row_adds_ln2,
        pins.test_p7_affine_in_v_and_constant_v,
        pins.test_p8_gqa_equals_mha_on_repeated_kv_heads,
        lambda: pins.test_p9_combine_of_any_partition_equals_unsplit(0),
        pins.test_combine_closed_forms,
        pins.test_p10_mla_equals_gqa_with_materialised_value_copy,
        pins.test_p10_absorbed_equals_unabsorbed_attention,
        pins.test_p12_dominant_key_selects_its_value,
        lambda: pins.test_varlen_whole_prompt_equals_causal_sdpa(4, 2),
        lambda: pins.test_varlen_chunk_equals_tail_of_whole_prompt(3),
        pins.test_varlen_without_mask_equals_sdpa,
        pins.test_varlen_rows_that_see_no_key,
        pins.test_mla_varlen_equals_gqa_varlen_with_materialised_value,
    ]


def _build_mutant(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"lib_{name}.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-std=c11", "-o", str(so_path), str(c_path), "-lm"], check=True)
    return str(so_path)


def test_unmutated_oracle_passes_battery():
    for pin in _battery():
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = oracle.load_library(_build_mutant(tmp_path, name, old, new))
    saved = oracle._lib
    oracle._lib = lib
    caught = []
    try:
        for pin in _battery():
            try:
                with np.errstate(all="ignore"):
                    pin()
            except (AssertionError, ValueError):
                caught.append(pin)
    finally:
        oracle._lib = saved
    assert caught, f"no pin caught mutant {name}"
