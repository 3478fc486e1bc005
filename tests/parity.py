"""Tolerances and comparison helpers for the GPU-vs-oracle parity tests.

Bars (stated once, used everywhere):
* out, float32 inputs:  max |gpu - oracle| <= 1e-5.
* out, bfloat16 inputs: |gpu - oracle| <= 2e-2 + 1e-2 |oracle| elementwise.
* lse (natural log, sink included): <= 1e-5 (float32) / 1e-3 (bfloat16).
  Scores of bf16 inputs are exact products summed in fp32, so the row
  log-sum-exp is far tighter than the bf16-rounded output.
* gradients (dq, dk, dv; dsink), relative to the tensor's scale:
  |gpu - oracle| <= c (rms(oracle) + |oracle|) elementwise, with
  c = 1e-4 (float32) and, for bfloat16 inputs, c = 5e-2 for dq/dk/dv and
  1e-2 for dsink.  The bf16 path feeds P and dS to the matrix cores as
  bf16 (as the forward feeds P), takes D_i = dO.O from the forward's
  bf16-rounded O, and rounds the gradients to bf16.  An fp64 evaluation of
  the backward with exactly those rounding points and nothing else
  (tests/test_backward_rounding.py) lands at about 3e-2 of this scale on
  the 1000-token, 64-head case; the bar leaves room for fp32 summation order
  only.  A wrong or missing term moves the result by the order of the scale
  itself.  Far from N(0,1) scale (queries x4, keys ramped to x4) the
  rounding of O alone moves dq to 7.4e-2 of the scale in that model; those
  cases use max(5e-2, 1.25 x the model's error on their own inputs).  Each check also records the worst error against the
  elementwise bar 2e-2 + 1e-2 |oracle| of the outputs, for the report
  printed at the end of the run.
"""
from __future__ import annotations

import numpy as np
import torch

OUT_F32_ATOL = 1e-5
OUT_BF16_ATOL, OUT_BF16_RTOL = 2e-2, 1e-2
LSE_ATOL = {torch.float32: 1e-5, torch.bfloat16: 1e-3}
GRAD_C = {torch.float32: 1e-4, torch.bfloat16: 5e-2}
DSINK_C = {torch.float32: 1e-4, torch.bfloat16: 1e-2}

# (what, dtype, worst err / (rms + |ref|), its bar, worst err / (2e-2 + 1e-2 |ref|),
#  worst abs err, rms(ref)) of every gradient check in this run
GRAD_REPORT: list = []


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
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(g - r))
    worst = float(np.nanmax(err)) if err.size else 0.0
    assert not np.isnan(err).any() and worst <= LSE_ATOL[dtype], \
        "%s: max abs err %.3g > %.1g" % (what, worst, LSE_ATOL[dtype])
    return worst


def check_out_nonfinite(gpu, ref, dtype, what="out", may_spread=None):
    """NaN-aware form of check_out for inputs holding NaN: every element the
    oracle gives as NaN must be NaN on the GPU too, every other element must
    be finite and within the bar.  ``may_spread`` (a boolean array of the
    same shape, or None) marks elements the GPU may additionally turn into
    NaN (a non-finite value row shared with them through a zero-weighted
    product); outside it the NaN patterns must be identical."""
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    rn, gn = np.isnan(r), np.isnan(g)
    missing = rn & ~gn
    assert not missing.any(), "%s: %d oracle NaN elements are not NaN on the GPU" % (
        what, int(missing.sum()))
    extra = gn & ~rn
    if may_spread is not None:
        extra &= ~np.asarray(may_spread, bool)
    assert not extra.any(), "%s: %d elements NaN on the GPU only" % (what, int(extra.sum()))
    keep = ~(rn | gn)
    assert np.isfinite(r[keep]).all() and np.isfinite(g[keep]).all(), "%s: infinities" % what
    return check_out(g[keep], r[keep], dtype, what) if keep.any() else 0.0


def check_lse_nonfinite(gpu, ref, dtype, what="lse"):
    """check_lse with identical NaN patterns required."""
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    rn, gn = np.isnan(r), np.isnan(g)
    assert np.array_equal(rn, gn), "%s: NaN patterns differ (%d oracle, %d GPU)" % (
        what, int(rn.sum()), int(gn.sum()))
    return check_lse(g[~rn], r[~rn], dtype, what) if (~rn).any() else 0.0


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
    plain = err / (OUT_BF16_ATOL + OUT_BF16_RTOL * np.abs(r))
    GRAD_REPORT.append((what, str(dtype).replace("torch.", ""), worst, c,
                        float(plain.max()) if plain.size else 0.0, float(err.max()) if err.size else 0.0,
                        rms))
    assert worst <= c, "%s: max err/(rms+|ref|) %.3g > %.1g (max abs err %.3g, rms %.3g)" % (
        what, worst, c, float(err.max()), rms)
    return worst
