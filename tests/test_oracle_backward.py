"""Pins of the oracle's attention backward against things other than itself
(CPU only).

The backward is tied to
* torch autograd through a plain float64 forward written with library ops
  (the sink as one extra virtual key of logit s_h and value 0, softmax, matmul),
* central finite differences of the loss computed with the oracle's own,
  separately pinned forward,
* invariants: GQA equals multi-head attention over repeat-interleaved K/V with
  dK/dV summed over each group; the sink gradient equals
  -sum_i e^{s_h - lse_i} (dO_i . O_i) evaluated with forward outputs; a sink
  of -inf has zero gradient.
Shapes are asymmetric (B > 1, Hq != Hkv, S != D, odd windows) so that a
swapped index or a dropped term fails at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from tests.sdpa_ref import band_mask


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def case(B=2, S=23, Hq=6, Hkv=2, D=8, seed=0):
    q = rnd((B, S, Hq, D), seed, 1.5)
    k = rnd((B, S, Hkv, D), seed + 1, 1.5)
    v = rnd((B, S, Hkv, D), seed + 2)
    sink = rnd((Hq,), seed + 3)
    dout = rnd((B, S, Hq, D), seed + 4)
    return q, k, v, sink, dout


def autograd_grads(q, k, v, sink, dout, W):
    """d(sum(dout * out))/d(q, k, v, sink) by torch autograd through a plain
    float64 forward: softmax over the window's keys and one virtual key whose
    logit is s_h and whose value vector is zero."""
    q, k, v, sink = (torch.tensor(np.asarray(a, np.float64), requires_grad=True)
                     for a in (q, k, v, sink))
    g = torch.as_tensor(np.asarray(dout, np.float64))
    B, S, Hq, D = q.shape
    G = Hq // k.shape[2]
    qh = q.permute(0, 2, 1, 3)
    kh = k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vh = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    logits = torch.matmul(qh, kh.transpose(-1, -2).contiguous()) / math.sqrt(D)
    allowed = torch.as_tensor(band_mask(S, W))
    logits = logits.masked_fill(~allowed, -math.inf)
    sink_col = sink[None, :, None, None].expand(B, Hq, S, 1)
    p = torch.softmax(torch.cat([logits, sink_col], dim=-1), dim=-1)
    out = torch.matmul(p[..., :S], vh).permute(0, 2, 1, 3)
    loss = (out * g).sum()
    return [t.numpy() for t in torch.autograd.grad(loss, [q, k, v, sink])]


@pytest.mark.parametrize("W", [1, 4, 9, 23, 100])
def test_backward_equals_autograd(W):
    q, k, v, sink, dout = case()
    got = oracle.attend_backward(q, k, v, sink, dout, W)
    ref = autograd_grads(q, k, v, sink, dout, W)
    for name, a, b in zip(("dq", "dk", "dv", "dsink"), got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11, err_msg=name)


def test_backward_equals_autograd_gqa_shapes():
    q, k, v, sink, dout = case(B=1, S=41, Hq=8, Hkv=1, D=16, seed=5)
    got = oracle.attend_backward(q, k, v, sink, dout, 17)
    ref = autograd_grads(q, k, v, sink, dout, 17)
    for name, a, b in zip(("dq", "dk", "dv", "dsink"), got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11, err_msg=name)


def test_sink_neg_inf_has_zero_gradient():
    q, k, v, sink, dout = case(seed=7)
    sink[::2] = -np.inf
    dq, dk, dv, dsink = oracle.attend_backward(q, k, v, sink, dout, 9)
    assert np.all(dsink[::2] == 0.0)
    ref = autograd_grads(q, k, v, sink, dout, 9)
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11, err_msg=name)


def test_backward_matches_finite_differences():
    """Every parameter of a tiny case: central differences of
    L = sum(dout * out) with out from the oracle's forward."""
    B, S, Hq, Hkv, D, W = 1, 7, 4, 2, 3, 4
    q, k, v, sink, dout = case(B, S, Hq, Hkv, D, seed=11)
    grads = oracle.attend_backward(q, k, v, sink, dout, W)
    params = [q, k, v, sink]

    def loss():
        out, _ = oracle.swa_prefill(q, k, v, sink, W)
        return float((out * dout).sum())

    h = 1e-5
    for p, g in zip(params, grads):
        flat, gflat = p.reshape(-1), g.reshape(-1)
        for e in range(flat.size):
            x0 = flat[e]
            flat[e] = x0 + h
            lp = loss()
            flat[e] = x0 - h
            lm = loss()
            flat[e] = x0
            assert abs((lp - lm) / (2 * h) - gflat[e]) <= 1e-7, (e, gflat[e])


def test_gqa_is_repeated_kv_heads_summed():
    q, k, v, sink, dout = case(B=2, S=19, Hq=6, Hkv=3, D=5, seed=13)
    G = 2
    dq, dk, dv, ds = oracle.attend_backward(q, k, v, sink, dout, 6)
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    dq2, dk2, dv2, ds2 = oracle.attend_backward(q, kr, vr, sink, dout, 6)
    B, S, Hkv, D = k.shape
    np.testing.assert_allclose(dq, dq2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ds, ds2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(B, S, Hkv, G, D).sum(3), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(B, S, Hkv, G, D).sum(3), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("W", [3, 23])
def test_sink_gradient_from_forward_outputs(W):
    """ds_h = -sum_{b,i} e^{s_h - lse_i} (dO_i . O_i), with O and lse from the
    oracle's forward (the sink's value vector is zero)."""
    q, k, v, sink, dout = case(seed=17)
    out, lse = oracle.swa_prefill(q, k, v, sink, W)               # lse [B, Hq, S]
    dot = (dout * out).sum(-1).transpose(0, 2, 1)                 # [B, Hq, S]
    expect = -(np.exp(sink[None, :, None] - lse) * dot).sum(axis=(0, 2))
    _, _, _, dsink = oracle.attend_backward(q, k, v, sink, dout, W)
    np.testing.assert_allclose(dsink, expect, rtol=1e-11, atol=1e-12)


def test_dv_is_attention_weights_times_dout():
    """With a single query head, dV_j = sum_i P_ij dO_i where P comes from the
    forward as softmax weights recovered from out (V = identity rows)."""
    B, S, Hq, Hkv, D, W = 1, 6, 1, 1, 6, 4
    q, k, _, sink, dout = case(B, S, Hq, Hkv, D, seed=19)
    v = np.eye(S)[None, :, None, :]                               # v_j = e_j
    out, _ = oracle.swa_prefill(q, k, v, sink, W)                  # out_i = P_i.
    P = out[0, :, 0, :]                                            # [i, j]
    _, _, dv, _ = oracle.attend_backward(q, k, v, sink, dout, W)
    np.testing.assert_allclose(dv[0, :, 0, :], P.T @ dout[0, :, 0, :], rtol=1e-12, atol=1e-13)
