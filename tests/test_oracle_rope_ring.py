"""Pins of the oracle's rotary embedding, ring append and ring decode with a
window shorter than the ring (CPU only).

RoPE (reading: dimension i paired with i + D/2, angle pos * theta^(-2i/D),
positions absolute -- ICML 2026 talk, Q&A on RoPE) is tied to
* torch complex arithmetic: (x_i + i x_{i+D/2}) * e^{i a} via torch.polar;
* invariants: position 0 is the identity, each pair keeps its norm, and
  <rope(q, m), rope(k, n)> depends only on m - n.
Ring decode with a window W in a ring of R slots is tied to the separately
pinned sliding-window prefill: stepping a sequence through append + decode
with MTP drafts (T tokens per step, a random number of them accepted and
the rest rolled back by resetting the length) reproduces, at every step and
for every draft, the prefill row of the sequence "accepted prefix + current
drafts" whenever R >= W + T - 1 -- and with R = W the drafts see shortened
windows, as the exact-window ring decode does.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle

TIGHT = dict(rtol=1e-12, atol=1e-12)


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def torch_rope(x, pos, theta):
    x = torch.as_tensor(np.asarray(x, np.float64))
    n, H, D = x.shape
    half = D // 2
    i = torch.arange(half, dtype=torch.float64)
    ang = torch.as_tensor(np.asarray(pos, np.float64))[:, None] * theta ** (-2.0 * i / D)
    z = torch.complex(x[..., :half], x[..., half:])
    r = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([r.real, r.imag], dim=-1).numpy()


@pytest.mark.parametrize("theta", [10000.0, 1e6])
def test_rope_equals_complex_rotation(theta):
    x = rnd((7, 3, 16), 1)
    pos = np.array([0, 1, 5, 127, 128, 4096, 262143])
    np.testing.assert_allclose(oracle.rope(x, pos, theta), torch_rope(x, pos, theta), rtol=1e-12,
                               atol=1e-12)


def test_rope_invariants():
    D, theta = 32, 10000.0
    q = rnd((1, 1, D), 2)
    k = rnd((1, 1, D), 3)
    np.testing.assert_array_equal(oracle.rope(q, [0], theta), q)
    y = oracle.rope(q, [777], theta)
    np.testing.assert_allclose(y[..., :16] ** 2 + y[..., 16:] ** 2,
                               q[..., :16] ** 2 + q[..., 16:] ** 2, **TIGHT)
    dots = []
    for shift in (0, 1, 1000, 123456):
        a = oracle.rope(q, [40 + shift], theta)
        b = oracle.rope(k, [9 + shift], theta)
        dots.append(float((a * b).sum()))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9, atol=1e-9)


def simulate(R, W, T, steps, seed, B=2, Hq=4, Hkv=2, D=8, theta=10000.0):
    """Run append + decode steps with random acceptance; return, per step, the
    decode output and the prefill rows of the reference sequence."""
    rng = np.random.default_rng(seed)
    sink = rng.standard_normal(Hq)
    kc = np.zeros((B, Hkv, R, D))
    vc = np.zeros((B, Hkv, R, D))
    L = np.zeros(B, dtype=np.int64)
    seq_q = [[] for _ in range(B)]          # post-RoPE rows of the accepted prefix
    seq_k = [[] for _ in range(B)]
    seq_v = [[] for _ in range(B)]
    results = []
    for _ in range(steps):
        q = rng.standard_normal((B, T, Hq, D))
        kn = rng.standard_normal((B, T, Hkv, D))
        vn = rng.standard_normal((B, T, Hkv, D))
        q_rot, kc, vc = oracle.rope_append(q, kn, vn, kc, vc, L, theta)
        out, lse = oracle.ring_decode(q_rot, kc, vc, sink, L + T, window=W)
        k_rot = oracle.rope(kn.reshape(B * T, Hkv, D),
                            (L[:, None] + np.arange(T)).reshape(-1), theta).reshape(B, T, Hkv, D)
        for b in range(B):
            fq = np.array(seq_q[b] + [q_rot[b, t] for t in range(T)])[None]
            fk = np.array(seq_k[b] + [k_rot[b, t] for t in range(T)])[None]
            fv = np.array(seq_v[b] + [vn[b, t] for t in range(T)])[None]
            ref, ref_lse = oracle.swa_prefill(fq, fk, fv, sink, W)
            results.append((out[b], lse[b], ref[0, -T:], ref_lse[0, :, -T:].T))
            acc = int(rng.integers(1, T + 1))            # the first token is always kept
            seq_q[b] += [q_rot[b, t] for t in range(acc)]
            seq_k[b] += [k_rot[b, t] for t in range(acc)]
            seq_v[b] += [vn[b, t] for t in range(acc)]
            L[b] += acc                                   # rejected drafts rolled back
    return results


@pytest.mark.parametrize("R,W,T", [(7, 5, 3), (10, 5, 3), (9, 9, 1)])
def test_rollback_ring_gives_full_windows(R, W, T):
    for out, lse, ref, ref_lse in simulate(R, W, T, steps=9, seed=R * 100 + W):
        np.testing.assert_allclose(out, ref, **TIGHT)
        np.testing.assert_allclose(lse, ref_lse, **TIGHT)


def test_exact_window_ring_shortens_draft_windows():
    """R = W = 5, T = 3: with no rollback room, the first drafts lose keys
    (the exact-window ring decode semantics), so some rows differ from the
    full-window prefill once the ring has wrapped."""
    res = simulate(5, 5, 3, steps=6, seed=7)
    assert any(not np.allclose(out, ref, rtol=1e-9, atol=1e-9) for out, _, ref, _ in res)


def test_window_equal_ring_matches_default():
    B, T, Hq, Hkv, W, D = 2, 2, 4, 2, 6, 8
    q = rnd((B, T, Hq, D), 11)
    kc = rnd((B, Hkv, W, D), 12)
    vc = rnd((B, Hkv, W, D), 13)
    sink = rnd((Hq,), 14)
    L = np.array([9, 4])
    a = oracle.ring_decode(q, kc, vc, sink, L)
    b = oracle.ring_decode(q, kc, vc, sink, L, window=W)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
