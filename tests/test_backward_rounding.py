"""Where the bf16 gradient bar comes from (CPU only).

The bf16 backward rounds at fixed points: the forward's output O (bf16, so
D_i = dO_i . O_i uses the rounded O), the probabilities P fed to the dV
product, P as handed (in fp16) to the wave that forms dS for dK, the score
gradients dS fed to the dQ and dK products, and the gradients themselves.  This test evaluates the backward in fp64 with exactly
those rounding points and no other error (numpy/torch, dense masked
matrices), and measures how far that moves the result from the exact fp64
oracle, in the unit the GPU tests use: |err| / (rms(ref) + |ref|).

That error is the floor any correct bf16 kernel with these rounding points
reaches; the GPU bar (5e-2) must sit above it with room for fp32 summation
order, and far below the O(1) a wrong term gives.  Source of the method: the
sink is a learnable per-head term of the softmax denominator
(technical-report digest, 前置知识 / 注意力sink偏置), so its gradient is part
of the result.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from sliding_window_learnable_amd import inputs
from tests.bf16_model import BF16, rb, rounded_backward, scaled_error
from tests.parity import GRAD_C, to64
from tests.test_gpu_dynamic_range import scaled_inputs


@pytest.mark.parametrize("S,Hq,Hkv,W", [(300, 8, 1, 128), (1000, 64, 8, 128)])
def test_rounding_points_set_the_bf16_gradient_floor(S, Hq, Hkv, W):
    D = 128
    q, k, v, sink = inputs.attention_inputs(70, 0, 1, S, S, Hq, Hkv, D, BF16)
    g = inputs.upstream_grad(70, 0, 1, S, Hq, D, BF16)
    q, k, v, sink, g = to64(q), to64(k), to64(v), to64(sink), to64(g)
    exact = oracle.attend_backward(q, k, v, sink, g, W)
    sim = rounded_backward(q, k, v, sink, g, W)
    errs = {n: scaled_error(a, r) for n, a, r in zip(("dq", "dk", "dv"), sim[:3], exact[:3])}
    print("rounding-point floor (S=%d, Hq=%d):" % (S, Hq),
          ", ".join("%s %.3g" % kv for kv in errs.items()))
    # the rounding alone must stay clearly below the bar ...
    assert max(errs.values()) < 0.8 * GRAD_C[BF16], errs
    # ... and be a real effect (the bar is not loose by orders of magnitude)
    assert max(errs.values()) > 0.1 * GRAD_C[BF16], errs
    # the simulation itself is the backward: without rounding it is the oracle
    plain = rounded_backward(q, k, v, sink, g, W, rnd=lambda x: x)
    for a, r in zip(plain, exact):
        assert np.abs(a - r).max() <= 1e-9 * (1 + np.abs(r).max())


def test_high_dynamic_range_floor_comes_from_the_rounded_output():
    """With queries x4 and key rows ramped x1..x4 (the GPU's high-dynamic-
    range backward case) the model's dq error passes the N(0,1) bar, and
    rounding O alone (D_i = dO.O from the bf16 output) accounts for it: the
    reason those GPU cases take the model's own floor as their bar."""
    S, Hq, Hkv, D, W = 300, 16, 2, 128, 128
    q, k, v, sink = scaled_inputs(135, 1, S, S, Hq, Hkv, D, q_scale=4.0)
    g = inputs.upstream_grad(135, 0, 1, S, Hq, D, BF16)
    args = (to64(q), to64(k), to64(v), to64(sink), to64(g), W)
    exact = oracle.attend_backward(*args)
    full = scaled_error(rounded_backward(*args)[0], exact[0])
    ident = lambda x: x                                          # noqa: E731
    only_o = rounded_backward(*args, rnd=ident, rnd_out=rb)
    print("dq floor: all rounding points %.3g, O alone %.3g" % (
        full, scaled_error(only_o[0], exact[0])))
    assert full > GRAD_C[BF16]
    assert scaled_error(only_o[0], exact[0]) > 0.9 * full
