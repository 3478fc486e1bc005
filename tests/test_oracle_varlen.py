"""Pins of the oracle's packed variable-length prefill (CPU only).

A packed batch is a block-diagonal problem: each sequence restarts its
positions at 0 and no row sees another sequence's keys.  The pins express
that through the library reference (one long sequence whose mask is the
block-diagonal band), through causality (right padding changes no real row)
and through independence (editing one sequence leaves the others alone).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.sdpa_ref import sdpa_with_sink

TIGHT = dict(rtol=1e-12, atol=1e-12)


def packed_case(lengths, Hq=6, Hkv=2, D=12, seed=0):
    rng = np.random.default_rng(seed)
    total = int(sum(lengths))
    q = rng.standard_normal((total, Hq, D)) * 1.5
    k = rng.standard_normal((total, Hkv, D)) * 1.5
    v = rng.standard_normal((total, Hkv, D))
    sink = rng.standard_normal(Hq)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q, k, v, sink, cu


def block_diagonal_band(cu, W):
    """Key j visible to query i iff both lie in one sequence and
    0 <= pos(i) - pos(j) < W, with positions counted from the sequence start."""
    total = int(cu[-1])
    seq = np.zeros(total, dtype=np.int64)
    pos = np.zeros(total, dtype=np.int64)
    for b in range(len(cu) - 1):
        seq[cu[b]:cu[b + 1]] = b
        pos[cu[b]:cu[b + 1]] = np.arange(cu[b + 1] - cu[b])
    d = pos[:, None] - pos[None, :]
    return (seq[:, None] == seq[None, :]) & (d >= 0) & (d < W)


LENGTHS = [[5, 0, 33, 1, 17], [40], [0, 9, 0], [12, 12, 12]]


@pytest.mark.parametrize("lengths", LENGTHS)
@pytest.mark.parametrize("W", [1, 4, 16, 1000])
def test_varlen_equals_sdpa_with_block_diagonal_mask(lengths, W):
    q, k, v, sink, cu = packed_case(lengths, seed=len(lengths) + W)
    out, lse = oracle.prefill_varlen(q, k, v, sink, cu, W)
    ref_out, ref_lse = sdpa_with_sink(q[None], k[None], v[None], sink,
                                      block_diagonal_band(cu, W)[None])
    np.testing.assert_allclose(out, ref_out[0], **TIGHT)
    np.testing.assert_allclose(lse, ref_lse[0], **TIGHT)


def test_block_diagonal_mask_tells_leakage_apart():
    """Treating the pack as one long sequence (positions not restarted, rows
    seeing the previous sequence) gives a visibly different result."""
    q, k, v, sink, cu = packed_case([20, 30], seed=3)
    out, _ = oracle.prefill_varlen(q, k, v, sink, cu, 16)
    leaky, _ = oracle.swa_prefill(q[None], k[None], v[None], sink, 16)
    assert np.abs(out[20:24] - leaky[0, 20:24]).max() > 1e-3
    np.testing.assert_allclose(out[:20], leaky[0, :20], **TIGHT)   # first sequence alone


@pytest.mark.parametrize("W", [3, 64])
def test_right_padding_changes_no_real_row(W):
    """Causality: sequence b padded on the right to the longest length and run
    as a uniform batch gives the same first S_b rows."""
    lengths = [7, 26, 1, 19]
    q, k, v, sink, cu = packed_case(lengths, seed=11)
    out, lse = oracle.prefill_varlen(q, k, v, sink, cu, W)
    S = max(lengths)
    rng = np.random.default_rng(99)
    qp = rng.standard_normal((len(lengths), S) + q.shape[1:])
    kp = rng.standard_normal((len(lengths), S) + k.shape[1:])
    vp = rng.standard_normal((len(lengths), S) + v.shape[1:])
    for b, n in enumerate(lengths):
        qp[b, :n], kp[b, :n], vp[b, :n] = q[cu[b]:cu[b + 1]], k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]]
    ref_out, ref_lse = sdpa_with_sink(qp, kp, vp, sink,
                                      block_diagonal_band(np.array([0, S]), W)[None])
    for b, n in enumerate(lengths):
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref_out[b, :n], **TIGHT)
        np.testing.assert_allclose(lse[:, cu[b]:cu[b + 1]], ref_lse[b, :, :n], **TIGHT)


def test_sequences_are_independent():
    q, k, v, sink, cu = packed_case([10, 15, 8], seed=5)
    out, lse = oracle.prefill_varlen(q, k, v, sink, cu, 6)
    k2, v2 = k.copy(), v.copy()
    k2[10:25] += 3.0
    v2[10:25] -= 2.0
    out2, lse2 = oracle.prefill_varlen(q, k2, v2, sink, cu, 6)
    for s0, s1 in ((0, 10), (25, 33)):
        np.testing.assert_array_equal(out[s0:s1], out2[s0:s1])
        np.testing.assert_array_equal(lse[:, s0:s1], lse2[:, s0:s1])
    assert np.abs(out[10:25] - out2[10:25]).max() > 1e-3
