"""Pins of the oracle's block maxima of global causal attention logits
(CPU only).

The block score is the largest scaled logit q_i . k_j / sqrt(D) over the
visible pairs of a (32-row query block, block_k-key block), -inf when the
block sees nothing (the reading of the High Sparse block scores, ICML 2026
talk §02).  It is tied to
* torch: the full fp64 logit matrix from a library matmul, the bottom-right
  causal mask, blocks by reshaping, and amax;
* plain Python loops on a tiny case (no numpy arithmetic);
* the oracle's own separately pinned forward: with sink -inf, each row's
  max logit lies in [lse_i - ln(n_i), lse_i] (n_i visible keys);
* structure: with k = 0 every visible block is exactly 0 and the invisible
  ones are -inf, and query heads sharing a KV head with equal q agree.
Shapes are ragged (S_q, S_kv not multiples of the blocks, S_q < S_kv).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def torch_block_max(q, k, block_k):
    q = torch.as_tensor(np.asarray(q, np.float64))
    k = torch.as_tensor(np.asarray(k, np.float64))
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kh = k.repeat_interleave(G, dim=2).permute(0, 2, 3, 1).contiguous()   # [B, Hq, D, Skv]
    x = torch.matmul(q.permute(0, 2, 1, 3), kh) / math.sqrt(D)             # [B, Hq, Sq, Skv]
    pos = torch.arange(Skv - Sq, Skv)[:, None]
    x = x.masked_fill(torch.arange(Skv)[None, :] > pos, -math.inf)
    nqb, nkb = -(-Sq // 32), -(-Skv // block_k)
    pad = torch.full((B, Hq, nqb * 32, nkb * block_k), -math.inf, dtype=torch.float64)
    pad[:, :, :Sq, :Skv] = x
    return pad.reshape(B, Hq, nqb, 32, nkb, block_k).amax(dim=(3, 5)).numpy()


@pytest.mark.parametrize("Sq,Skv,bk", [(70, 70, 32), (70, 90, 64), (33, 200, 96), (1, 50, 32)])
def test_block_max_equals_torch(Sq, Skv, bk):
    q = rnd((2, Sq, 4, 16), 1)
    k = rnd((2, Skv, 2, 16), 2)
    got = oracle.block_max(q, k, bk)
    ref = torch_block_max(q, k, bk)
    assert got.shape == ref.shape
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_block_max_brute_force_loops():
    B, Sq, Skv, Hq, Hkv, D, bk = 1, 35, 40, 2, 1, 3, 8
    q = rnd((B, Sq, Hq, D), 3)
    k = rnd((B, Skv, Hkv, D), 4)
    got = oracle.block_max(q, k, bk)
    for h in range(Hq):
        for qb in range(got.shape[2]):
            for kb in range(got.shape[3]):
                best = -math.inf
                for i in range(32 * qb, min(Sq, 32 * qb + 32)):
                    for j in range(kb * bk, min(Skv, kb * bk + bk)):
                        if j <= Skv - Sq + i:
                            x = sum(float(q[0, i, h, d]) * float(k[0, j, 0, d]) for d in range(D))
                            best = max(best, x / math.sqrt(D))
                if best == -math.inf:
                    assert got[0, h, qb, kb] == -math.inf
                else:
                    assert abs(got[0, h, qb, kb] - best) <= 1e-12


def test_row_max_brackets_lse():
    """sink = -inf: lse_i = ln sum_j e^{x_ij}, so max_j x_ij is in
    [lse_i - ln(n_i), lse_i]; the row block's max over its key blocks is the
    max over its rows of max_j x_ij."""
    B, Sq, Skv, Hq, Hkv, D = 1, 64, 100, 2, 1, 8
    q = rnd((B, Sq, Hq, D), 5) * 2.0
    k = rnd((B, Skv, Hkv, D), 6)
    v = rnd((B, Skv, Hkv, D), 7)
    _, lse = oracle.global_attn(q, k, v, np.full(Hq, -np.inf))     # [B, Hq, Sq]
    bm = oracle.block_max(q, k, 16)
    n = np.arange(Skv - Sq, Skv) + 1                               # visible keys per row
    for h in range(Hq):
        for qb in range(2):
            rows = slice(32 * qb, 32 * qb + 32)
            top = bm[0, h, qb].max()
            assert top <= lse[0, h, rows].max() + 1e-12
            assert top >= (lse[0, h, rows] - np.log(n[rows])).max() - 1e-12


def test_zero_keys_give_the_causal_block_pattern():
    B, Sq, Skv, Hq, Hkv, D, bk = 1, 70, 100, 2, 2, 4, 16
    q = rnd((B, Sq, Hq, D), 8)
    k = np.zeros((B, Skv, Hkv, D))
    bm = oracle.block_max(q, k, bk)
    for qb in range(bm.shape[2]):
        last_pos = Skv - Sq + min(Sq - 1, 32 * qb + 31)
        for kb in range(bm.shape[3]):
            expect = 0.0 if kb * bk <= last_pos else -np.inf
            assert np.all(bm[0, :, qb, kb] == expect), (qb, kb)


def test_heads_of_a_group_with_equal_queries_agree():
    B, Sq, Skv, Hq, Hkv, D = 1, 40, 40, 4, 2, 8
    q = rnd((B, Sq, Hq, D), 9)
    q[:, :, 1] = q[:, :, 0]          # heads 0, 1 share KV head 0
    q[:, :, 3] = q[:, :, 0]          # head 3 uses KV head 1
    k = rnd((B, Skv, Hkv, D), 10)
    bm = oracle.block_max(q, k, 8)
    assert np.array_equal(bm[0, 0], bm[0, 1])
    assert not np.array_equal(bm[0, 0], bm[0, 3])
