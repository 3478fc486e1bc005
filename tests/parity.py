"""Tolerances and comparison helpers for the GPU-vs-oracle parity tests.

Bars (stated once, used everywhere):
* out, float32 inputs:  max |gpu - oracle| <= 1e-5.
* out, bfloat16 inputs: |gpu - oracle| <= 2e-2 + 1e-2 |oracle| elementwise.
* lse (natural log, sink included): <= 1e-5 (float32) / 1e-3 (bfloat16).
  Scores of bf16 inputs are exact products summed in fp32, so the row
  log-sum-exp is far tighter than the bf16-rounded output.
* gradients (dq, dk, dv; dsink), relative to the tensor's scale:
  |gpu - oracle| <= c (rms(oracle) + |oracle|) elementwise, with
  c = 1e-4 (float32) and, for bfloat16 inputs, c = 8e-2 for dq/dk/dv and
  1e-2 for dsink.  The bf16 path feeds P and dS to the matrix cores as
  bf16 (as the forward feeds P), and takes D_i = dO.O from the forward's
  bf16-rounded O.  Rounding P alone, evaluated exactly in fp64 on the
  1000-token, 64-head case, already moves dv by up to 2.8e-2 of this scale
  (the kernels measure 2-4.3e-2); a wrong or missing term moves the result
  by the order of the scale itself.
"""
from __future__ import annotations

import numpy as np
import torch

OUT_F32_ATOL = 1e-5
OUT_BF16_ATOL, OUT_BF16_RTOL = 2e-2, 1e-2
LSE_ATOL = {torch.float32: 1e-5, torch.bfloat16: 1e-3}
GRAD_C = {torch.float32: 1e-4, torch.bfloat16: 8e-2}
DSINK_C = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


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


def check_grad(gpu, ref, dtype, what, c=None):
    """|gpu - ref| <= c (rms(ref) + |ref|) elementwise (see the module notes)."""
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), "%s has non-finite values" % what
    if c is None:
        c = DSINK_C[dtype] if what == "dsink" else GRAD_C[dtype]
    rms = float(np.sqrt((r ** 2).mean())) if r.size else 0.0
    err = np.abs(g - r)
    ratio = err / (rms + np.abs(r) + 1e-30)
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= c, "%s: max err/(rms+|ref|) %.3g > %.1g (max abs err %.3g, rms %.3g)" % (
        what, worst, c, float(err.max()), rms)
    return worst
