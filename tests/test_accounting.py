"""FLOP/byte accounting used by the bench agrees with pairs enumerated by the
oracle, and reproduces the hybrid-stack reductions the pages quote (CPU)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from sliding_window_learnable_amd import accounting as acc


@pytest.mark.parametrize("S,W", [(1, 128), (127, 128), (128, 128), (129, 128), (32768, 128),
                                 (1000, 1), (70, 300)])
def test_window_pairs_match_oracle_enumeration(S, W):
    assert acc.window_pairs(S, W) == oracle.count_window_pairs(S, W)


def test_causal_pairs_is_window_ge_S():
    for S in (1, 2, 77, 4096):
        assert acc.causal_pairs(S, S) == oracle.count_window_pairs(S, S)
    # queries at the end of a longer sequence: rows see S_kv - S_q + i + 1 keys
    assert acc.causal_pairs(3, 10) == 8 + 9 + 10


def test_ring_pairs_full_ring_drafts():
    # full ring: draft t sees W - (T-1-t) keys
    assert acc.ring_pairs(4, 128, 10_000) == 125 + 126 + 127 + 128
    assert acc.ring_pairs(1, 128, 128) == 128
    assert acc.ring_pairs(4, 128, 2) == 0 + 0 + 1 + 2


def test_prefill_32k_counts():
    flops = acc.prefill_flops(1, 32768, 64, 128, 128)
    assert flops == 4 * 128 * 64 * (128 * 32768 - 128 * 127 // 2)
    assert abs(flops - 1.3717e11) / 1.3717e11 < 1e-3
    assert acc.prefill_bytes(1, 32768, 64, 8, 128) == (512 + 64 + 64 + 512 + 8) * 2**20


def test_hybrid_reductions_near_pages_six_fold():
    """5 SWA (W=128) + 1 global layer at S=65536 vs 6 global layers: about
    6x less attention compute and KV cache, the figure the MiMo-V2 wiki
    page (关键架构决策) and the technical-report digest (核心方法) quote."""
    compute, kv = acc.hybrid_ratios(65536, 128, 5)
    assert 5.85 < compute < 5.95
    assert 5.9 < kv < 6.0
    # the plain formula gives 8x for a 7:1 schedule (the talk quotes 7x)
    compute7, _ = acc.hybrid_ratios(262144, 128, 7)
    assert 7.9 < compute7 < 8.0


def test_roofline_fraction_is_one_at_the_bound():
    """At the ideal time of the binding resource the fraction is exactly 1:
    HBM for the 32K window-128 prefill (AI ~ 113 flop/B), MFMA for the 64K
    global layer."""
    f = acc.prefill_flops(1, 32768, 64, 128, 128)
    b = acc.prefill_bytes(1, 32768, 64, 8, 128)
    assert abs(acc.roofline_frac(f, b, b / (acc.PEAK_HBM_GBS * 1e9)) - 1.0) < 1e-12
    assert abs(acc.roofline_frac(f, b, 2 * b / (acc.PEAK_HBM_GBS * 1e9)) - 0.5) < 1e-12
    f = acc.global_flops(1, 65536, 65536, 64, 128)
    b = acc.global_bytes(1, 65536, 65536, 64, 8, 128)
    assert abs(acc.roofline_frac(f, b, f / (acc.PEAK_BF16_TFLOPS * 1e12)) - 1.0) < 1e-12
