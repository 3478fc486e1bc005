"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test ties the oracle to a library routine, a closed form, an invariant
or a high-precision brute force.  Shapes are deliberately asymmetric
(B > 1, Hq != Hkv, S != D, odd windows) so that a swapped index, a dropped
term or a wrong sign in the oracle fails at least one of them.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from tests.sdpa_ref import band_mask, causal_bottom_right, sdpa_with_sink

TIGHT = dict(rtol=1e-12, atol=1e-12)


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def tiny_case(B=2, S=37, Hq=6, Hkv=2, D=12, seed=0, qscale=1.5):
    q = rnd((B, S, Hq, D), seed, qscale)
    k = rnd((B, S, Hkv, D), seed + 1, qscale)
    v = rnd((B, S, Hkv, D), seed + 2)
    sink = rnd((Hq,), seed + 3)
    return q, k, v, sink


# --- the sink is a virtual token with logit s_h and value 0 -------------------

@pytest.mark.parametrize("W", [1, 5, 16, 37, 100])
def test_prefill_equals_sdpa_with_virtual_sink_token(W):
    q, k, v, sink = tiny_case()
    out, lse = oracle.swa_prefill(q, k, v, sink, W)
    ref_out, ref_lse = sdpa_with_sink(q, k, v, sink, band_mask(q.shape[1], W)[None])
    np.testing.assert_allclose(out, ref_out, **TIGHT)
    np.testing.assert_allclose(lse, ref_lse, **TIGHT)


def test_sink_scale_and_sign_matter():
    """A sink that is scaled by 1/sqrt(D), negated or shared across heads gives
    a different result: the library reference tells these readings apart."""
    q, k, v, sink = tiny_case(seed=7)
    out, _ = oracle.swa_prefill(q, k, v, sink, 9)
    mask = band_mask(q.shape[1], 9)[None]
    for wrong in (sink / math.sqrt(q.shape[-1]), -sink, np.full_like(sink, sink[0])):
        ref_wrong, _ = sdpa_with_sink(q, k, v, wrong, mask)
        assert np.abs(out - ref_wrong).max() > 1e-3


# --- config-1 reductions (tiny reference: B=1, H=1, S=512, D=64, W=128) --------

def config1(seed=1001):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 512, 1, 64))
    k = rng.standard_normal((1, 512, 1, 64))
    v = rng.standard_normal((1, 512, 1, 64))
    sink = rng.standard_normal((1,))
    return q, k, v, sink


def test_sink_neg_inf_is_banded_softmax_attention():
    q, k, v, _ = config1()
    sink = np.array([-np.inf])
    out, lse = oracle.swa_prefill(q, k, v, sink, 128)
    import torch
    import torch.nn.functional as F
    qh, kh, vh = (torch.as_tensor(a).permute(0, 2, 1, 3) for a in (q, k, v))
    ref = F.scaled_dot_product_attention(qh, kh, vh,
                                         attn_mask=torch.as_tensor(band_mask(512, 128)))
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), **TIGHT)
    logits = torch.matmul(qh, kh.transpose(-1, -2).contiguous()) / 8.0
    logits = logits.masked_fill(~torch.as_tensor(band_mask(512, 128)), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).numpy(), **TIGHT)


def test_window_ge_S_is_full_causal_attention():
    q, k, v, sink = config1()
    import torch
    import torch.nn.functional as F
    qh, kh, vh = (torch.as_tensor(a).permute(0, 2, 1, 3) for a in (q, k, v))
    causal = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True)
    out, _ = oracle.swa_prefill(q, k, v, np.array([-np.inf]), 512)
    np.testing.assert_allclose(out, causal.permute(0, 2, 1, 3).numpy(), **TIGHT)
    # a window larger than the sequence changes nothing; the global call agrees
    out_w, lse_w = oracle.swa_prefill(q, k, v, sink, 512)
    out_big, lse_big = oracle.swa_prefill(q, k, v, sink, 10_000)
    out_g, lse_g = oracle.global_attn(q, k, v, sink)
    assert np.array_equal(out_w, out_big) and np.array_equal(lse_w, lse_big)
    np.testing.assert_allclose(out_g, out_w, **TIGHT)
    np.testing.assert_allclose(lse_g, lse_w, **TIGHT)
    ref, ref_lse = sdpa_with_sink(q, k, v, sink, band_mask(512, 512)[None])
    np.testing.assert_allclose(out_w, ref, **TIGHT)
    np.testing.assert_allclose(lse_w, ref_lse, **TIGHT)


# --- closed forms ---------------------------------------------------------------

def test_real_token_mass_is_one_minus_sink_share():
    """With every value vector equal to 1 the output is the attention mass on
    real tokens: Z/(Z+e^s) = 1 - exp(s - lse), strictly below 1."""
    q, k, v, sink = tiny_case(seed=11)
    v = np.ones_like(v)
    out, lse = oracle.swa_prefill(q, k, v, sink, 7)
    share = np.exp(sink[None, :, None] - lse)                     # B Hq S
    expect = 1.0 - share.transpose(0, 2, 1)[..., None]
    np.testing.assert_allclose(out, np.broadcast_to(expect, out.shape), **TIGHT)
    assert (out < 1.0).all() and (out > 0.0).all()
    # sink -> -inf puts all mass back on the real tokens
    out_inf, _ = oracle.swa_prefill(q, k, v, np.full_like(sink, -np.inf), 7)
    np.testing.assert_allclose(out_inf, 1.0, **TIGHT)


def test_single_key_is_logistic():
    """Window 1 (and row 0 for any window): one real key against the sink,
    out = sigmoid(x_ii - s) v_i and lse = log(e^{x_ii} + e^s)."""
    q, k, v, sink = tiny_case(seed=21)
    B, S, Hq, D = q.shape
    G = Hq // k.shape[2]
    kk = np.repeat(k, G, axis=2)
    vv = np.repeat(v, G, axis=2)
    x = (q * kk).sum(-1) / math.sqrt(D)                          # B S Hq
    sig = 1.0 / (1.0 + np.exp(-(x - sink[None, None, :])))
    out1, lse1 = oracle.swa_prefill(q, k, v, sink, 1)
    np.testing.assert_allclose(out1, sig[..., None] * vv, **TIGHT)
    np.testing.assert_allclose(lse1, np.logaddexp(x, sink).transpose(0, 2, 1), **TIGHT)
    out9, lse9 = oracle.swa_prefill(q, k, v, sink, 9)
    np.testing.assert_allclose(out9[:, 0], sig[:, 0, :, None] * vv[:, 0], **TIGHT)
    np.testing.assert_allclose(lse9[:, :, 0], np.logaddexp(x[:, 0], sink), **TIGHT)


# --- invariants -------------------------------------------------------------------

def test_window_locality():
    """Keys older than i-W+1 and keys after i do not influence row i (bitwise)."""
    q, k, v, sink = tiny_case(seed=31, S=40)
    W, i = 6, 20
    out, lse = oracle.swa_prefill(q, k, v, sink, W)
    k2, v2 = k.copy(), v.copy()
    outside = [j for j in range(40) if j < i - W + 1 or j > i]
    k2[:, outside] = rnd(k2[:, outside].shape, 99, 5.0)
    v2[:, outside] = rnd(v2[:, outside].shape, 98, 5.0)
    out2, lse2 = oracle.swa_prefill(q, k2, v2, sink, W)
    assert np.array_equal(out[:, i], out2[:, i])
    assert np.array_equal(lse[:, :, i], lse2[:, :, i])
    assert not np.allclose(out[:, i + 1], out2[:, i + 1])        # row i+1 does see j=i+1


def test_gqa_head_mapping():
    """Query head h reads KV head h // (Hq/Hkv): moving one KV head changes
    exactly that group's outputs."""
    q, k, v, sink = tiny_case(seed=41, Hq=6, Hkv=3)
    out, _ = oracle.swa_prefill(q, k, v, sink, 8)
    k2 = k.copy()
    k2[:, :, 1] += 0.5
    out2, _ = oracle.swa_prefill(q, k2, v, sink, 8)
    changed = [h for h in range(6) if not np.array_equal(out[:, :, h], out2[:, :, h])]
    assert changed == [2, 3]


# --- brute force in 40-digit decimal arithmetic, keys in the outer loop ---------

def test_brute_force_decimal():
    getcontext().prec = 40
    B, S, Hq, Hkv, D, W = 1, 9, 2, 1, 3, 4
    q, k, v, sink = tiny_case(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, seed=51)
    sink[1] = -2.5
    out, lse = oracle.swa_prefill(q, k, v, sink, W)
    inv = Decimal(1) / Decimal(D).sqrt()
    num = {}
    den = {}
    for j in range(S):                                             # keys outer
        for h in range(Hq):
            for i in range(j, min(S, j + W)):                      # rows that see key j
                x = sum(Decimal(q[0, i, h, d]) * Decimal(k[0, j, 0, d]) for d in range(D)) * inv
                e = x.exp()
                den[i, h] = den.get((i, h), Decimal(0)) + e
                acc = num.setdefault((i, h), [Decimal(0)] * D)
                for d in range(D):
                    acc[d] += e * Decimal(v[0, j, 0, d])
    for (i, h), acc in num.items():
        total = den[i, h] + Decimal(sink[h]).exp()
        for d in range(D):
            assert abs(float(acc[d] / total) - out[0, i, h, d]) <= 1e-13
        assert abs(float(total.ln()) - lse[0, h, i]) <= 1e-13


# --- global causal attention with S_q < S_kv (bottom-right alignment) -----------

def test_global_bottom_right_causal():
    q, k, v, sink = tiny_case(seed=61, S=30)
    qd = q[:, -5:]
    out, lse = oracle.global_attn(qd, k, v, sink)
    ref, ref_lse = sdpa_with_sink(qd, k, v, sink, causal_bottom_right(5, 30)[None])
    np.testing.assert_allclose(out, ref, **TIGHT)
    np.testing.assert_allclose(lse, ref_lse, **TIGHT)
    full, full_lse = oracle.global_attn(q, k, v, sink)
    np.testing.assert_allclose(out, full[:, -5:], **TIGHT)
    np.testing.assert_allclose(lse, full_lse[:, :, -5:], **TIGHT)


# --- ring decode ------------------------------------------------------------------

def ring_from_sequence(kseq, W, L):
    """Write positions 0..L-1 of kseq [B, L, Hkv, D] into a W-slot ring
    (slot = position mod W); returns [B, Hkv, W, D]."""
    B, _, Hkv, D = kseq.shape
    ring = np.full((B, Hkv, W, D), np.nan)
    for P in range(L):
        ring[:, :, P % W] = kseq[:, P]
    return ring


@pytest.mark.parametrize("L,T", [(16, 1), (16, 4), (23, 1), (23, 4), (61, 3), (9, 4), (4, 4)])
def test_ring_decode_equals_sdpa_over_sequence(L, T):
    W, B, Hq, Hkv, D = 16, 2, 4, 2, 8
    rng = np.random.default_rng(L * 10 + T)
    kseq = rng.standard_normal((B, L, Hkv, D))
    vseq = rng.standard_normal((B, L, Hkv, D))
    q = rng.standard_normal((B, T, Hq, D)) * 1.3
    sink = rng.standard_normal(Hq)
    kc = ring_from_sequence(kseq, W, L)
    vc = ring_from_sequence(vseq, W, L)
    if L < W:                      # unwritten slots must never be read
        kc = np.where(np.isnan(kc), 1e300, kc)
        vc = np.where(np.isnan(vc), 1e300, vc)
    out, lse = oracle.ring_decode(q, kc, vc, sink, np.full(B, L))
    pos = L - T + np.arange(T)[:, None]
    j = np.arange(L)[None, :]
    allowed = (j <= pos) & (j >= max(0, L - W))
    ref, ref_lse = sdpa_with_sink(q, kseq, vseq, sink, allowed[None])
    np.testing.assert_allclose(out, ref, **TIGHT)
    np.testing.assert_allclose(lse, ref_lse.transpose(0, 2, 1), **TIGHT)


def test_ring_decode_full_ring_matches_prefill_and_is_slot_order_free():
    W, B, Hq, Hkv, D, S = 12, 2, 4, 2, 8, 12
    q, k, v, sink = tiny_case(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, seed=71)
    pre, pre_lse = oracle.swa_prefill(q, k, v, sink, W)
    kc = np.ascontiguousarray(k.transpose(0, 2, 1, 3))                 # slot = position
    vc = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    dec, dec_lse = oracle.ring_decode(q[:, -1:], kc, vc, sink)          # cache_len None: L = W
    np.testing.assert_allclose(dec[:, 0], pre[:, -1], **TIGHT)
    np.testing.assert_allclose(dec_lse[:, 0], pre_lse[:, :, -1], **TIGHT)
    perm = np.random.default_rng(3).permutation(W)
    dec_p, _ = oracle.ring_decode(q[:, -1:], kc[:, :, perm], vc[:, :, perm], sink)
    np.testing.assert_allclose(dec_p, dec, **TIGHT)


def test_ring_decode_draft_windows():
    """With a full ring, draft t sees W - (T-1-t) keys: the prefill row at the
    same position with that shorter window; the last draft sees the full W."""
    W, T, L, B, Hq, Hkv, D = 10, 4, 25, 1, 2, 1, 6
    q, k, v, sink = tiny_case(B=B, S=L, Hq=Hq, Hkv=Hkv, D=D, seed=81)
    kc = ring_from_sequence(k, W, L)
    vc = ring_from_sequence(v, W, L)
    dec, _ = oracle.ring_decode(q[:, -T:], kc, vc, sink, np.full(B, L))
    for t in range(T):
        pre, _ = oracle.swa_prefill(q, k, v, sink, W - (T - 1 - t))
        np.testing.assert_allclose(dec[:, t], pre[:, L - T + t], **TIGHT)


def test_ring_decode_empty_key_set_leaves_only_sink():
    W, B, Hq, Hkv, D = 8, 1, 2, 1, 4
    q, k, v, sink = tiny_case(B=B, S=3, Hq=Hq, Hkv=Hkv, D=D, seed=91)
    kc = np.zeros((B, Hkv, W, D))
    out, lse = oracle.ring_decode(q, kc, kc, sink, np.array([1]))     # L=1 < T=3
    assert np.all(out[:, :2] == 0.0)
    np.testing.assert_array_equal(lse[:, :2], np.broadcast_to(sink, (1, 2, Hq)))


# --- layer-level counts ----------------------------------------------------------

@pytest.mark.parametrize("S,W", [(1, 128), (100, 128), (128, 128), (129, 128), (5000, 128), (777, 1)])
def test_window_pair_count_closed_form(S, W):
    n = oracle.count_window_pairs(S, W)
    m = min(S, W)
    assert n == m * (m + 1) // 2 + max(0, S - W) * W
    if S >= W:
        assert n == W * S - W * (W - 1) // 2
