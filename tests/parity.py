"""Shared parity gate for GPU-vs-oracle comparisons.

Gate (fp16/bf16 outputs, fp32 accumulation on the GPU):
  * per element: |gpu - o64| <= 2e-3 + ulp(o64) / 2, i.e. 2e-3 of arithmetic
    error on top of the unavoidable rounding of the exact result to the output
    format (bf16's half-ulp alone is 3.9e-3 for |x| in [1, 2), which the
    literal 2e-3 cannot absorb);
  * RMS over all compared elements <= 5e-4 + RMS(round16(o64) - o64): the
    same 5e-4 of arithmetic error on top of the format's own rounding, which
    alone is about 0.29 ulp RMS (1.1e-3 for bf16 values in [0.5, 1));
  * lse (fp32): |gpu - o64| <= 2e-4 + 1e-6 |o64|  (fp32 scores and sums;
    -inf must match exactly).
The literal max-abs error is reported alongside.
"""
from __future__ import annotations

import math

import numpy as np
import torch

ABS_TOL = 2e-3
RMS_TOL = 5e-4
LSE_ABS = 2e-4
LSE_REL = 1e-6


def ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Spacing of the 16-bit format at |x| (x float64)."""
    mant = 10 if dtype == torch.float16 else 7
    emin = -14 if dtype == torch.float16 else -126
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - mant).astype(np.int64))


def gate(gpu_out: torch.Tensor, ref: np.ndarray, dtype: torch.dtype, gpu_lse=None, ref_lse=None,
         where: str = "") -> dict:
    g = gpu_out.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{where}: non-finite output"
    err = np.abs(g - ref)
    bound = ABS_TOL + 0.5 * ulp(ref, dtype)
    bad = err > bound
    rms = math.sqrt(float(np.mean(err ** 2))) if err.size else 0.0
    fmt = torch.from_numpy(ref).to(dtype).double().numpy() - ref
    rms_fmt = math.sqrt(float(np.mean(fmt ** 2))) if fmt.size else 0.0
    stats = {"max_abs": float(err.max()) if err.size else 0.0, "rms": rms, "rms_format": rms_fmt,
             "n_over_bound": int(bad.sum()), "n": int(err.size)}
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{where}: {stats['n_over_bound']} elements over bound; worst at {i}: "
                             f"gpu {g[i]!r} ref {ref[i]!r} bound {bound[i]:.3g}")
    assert rms <= RMS_TOL + rms_fmt, f"{where}: rms {rms:.3g} > {RMS_TOL} + {rms_fmt:.3g}"
    if gpu_lse is not None:
        gl = gpu_lse.detach().cpu().numpy().astype(np.float64)
        inf_ref = np.isneginf(ref_lse)
        assert np.array_equal(np.isneginf(gl), inf_ref), f"{where}: -inf lse pattern differs"
        fin = ~inf_ref
        lerr = np.abs(gl[fin] - ref_lse[fin])
        lb = LSE_ABS + LSE_REL * np.abs(ref_lse[fin])
        assert np.all(lerr <= lb), f"{where}: lse error {lerr.max():.3g}"
        stats["lse_max_abs"] = float(lerr.max()) if lerr.size else 0.0
    return stats
