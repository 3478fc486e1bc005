"""Tolerances and comparison helpers for the GPU-vs-oracle parity tests.

Bars (stated once, used everywhere):
* out, float32 inputs:  max |gpu - oracle| <= 1e-5.
* out, bfloat16 inputs: |gpu - oracle| <= 2e-2 + 1e-2 |oracle| elementwise.
* lse (natural log, sink included): <= 1e-5 (float32) / 1e-3 (bfloat16).
  Scores of bf16 inputs are exact products summed in fp32, so the row
  log-sum-exp is far tighter than the bf16-rounded output.
"""
from __future__ import annotations

import numpy as np
import torch

OUT_F32_ATOL = 1e-5
OUT_BF16_ATOL, OUT_BF16_RTOL = 2e-2, 1e-2
LSE_ATOL = {torch.float32: 1e-5, torch.bfloat16: 1e-3}


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def check_out(gpu, ref, dtype, what="out"):
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), "%s has non-finite values" % what
    err = np.abs(g - r)
    if dtype == torch.float32:
        worst = err.max() if err.size else 0.0
        assert worst <= OUT_F32_ATOL, "%s: max abs err %.3g > %.1g" % (what, worst, OUT_F32_ATOL)
    else:
        bound = OUT_BF16_ATOL + OUT_BF16_RTOL * np.abs(r)
        bad = err > bound
        assert not bad.any(), "%s: %d elements over 2e-2 + 1e-2|ref| (worst err %.3g)" % (
            what, int(bad.sum()), float(err.max()))
    return float(err.max()) if err.size else 0.0


def check_lse(gpu, ref, dtype, what="lse"):
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    same_inf = np.isinf(r) & (g == r)
    err = np.where(same_inf, 0.0, np.abs(g - r))
    worst = float(np.nanmax(err)) if err.size else 0.0
    assert not np.isnan(err).any() and worst <= LSE_ATOL[dtype], \
        "%s: max abs err %.3g > %.1g" % (what, worst, LSE_ATOL[dtype])
    return worst
