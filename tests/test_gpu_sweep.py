"""GPU parity over a seeded sweep of shapes, through the C ABI, against the
fp64 oracle: every bf16 entry point at shapes drawn from one fixed generator
(sequence lengths 1..700 with ragged tails, GQA groups 1..16 including odd
ones, D = 64 and 128, windows from 1 to past the sequence, decode rings
wider than the window, packed batches with empty sequences).  The shapes
are fixed by the seed, so a failure names a reproducible case."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.bf16_model import rounded_backward, scaled_error
from tests.parity import GRAD_C, check_grad, check_lse, check_out, to64

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
GROUPS = [(1, 1), (2, 1), (3, 1), (4, 2), (6, 2), (8, 1), (8, 4), (16, 2), (16, 1), (12, 4)]


def _cases(kind, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hq, Hkv = GROUPS[rng.integers(len(GROUPS))]
        D = int(rng.choice([64, 128]))
        if kind == "prefill":
            B = int(rng.integers(1, 4))
            S = int(rng.choice([rng.integers(1, 40), rng.integers(40, 700)]))
            W = int(rng.choice([1, 31, 98, 127, 128, 129, 200, 511, 10000, rng.integers(1, 800)]))
            out.append((i, B, S, Hq, Hkv, D, W))
        elif kind == "varlen":
            B = int(rng.integers(1, 7))
            lens = [int(x) for x in rng.choice([0, 1, 31, 32, 33, 100, 257, 600], size=B)]
            W = int(rng.choice([33, 128, 129, 300, 100000]))
            out.append((i, tuple(lens), Hq, Hkv, D, W))
        elif kind == "global":
            B = int(rng.integers(1, 3))
            Skv = int(rng.integers(1, 3000))
            Sq = int(min(Skv, rng.choice([1, 2, 4, 8, rng.integers(1, 200)])))
            out.append((i, B, Sq, Skv, Hq, Hkv, D))
        elif kind == "ring":
            B = int(rng.integers(1, 9))
            T = int(rng.integers(1, 5))
            W = int(rng.choice([T, 32, 100, 128]))
            W = max(W, T)
            R = W + int(rng.choice([0, T - 1, 17]))
            out.append((i, B, T, Hq, Hkv, D, W, R))
        else:  # backward
            S = int(rng.integers(1, 400))
            W = int(rng.choice([1, 33, 128, 200, 300, 100000]))
            out.append((i, 1, S, Hq, Hkv, D, W))
    return out


@pytest.mark.parametrize("i,B,S,Hq,Hkv,D,W", _cases("prefill", 16, 1001))
def test_prefill_sweep(gpu, i, B, S, Hq, Hkv, D, W):
    q, k, v, sink = inputs.attention_inputs(301, i, B, S, S, Hq, Hkv, D, BF16)
    ref_out, ref_lse = oracle.swa_prefill(to64(q), to64(k), to64(v), to64(sink), W)
    out, lse = swa.swa_sink_prefill(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu), W)
    torch.cuda.synchronize()
    check_out(out, ref_out, BF16)
    check_lse(lse, ref_lse, BF16)


@pytest.mark.parametrize("i,lens,Hq,Hkv,D,W", _cases("varlen", 10, 1002))
def test_varlen_sweep(gpu, i, lens, Hq, Hkv, D, W):
    if sum(lens) == 0:
        lens = lens[:-1] + (5,)
    q, k, v, sink, cu = inputs.packed_inputs(302, i, list(lens), Hq, Hkv, D, BF16)
    ref_out, ref_lse = oracle.prefill_varlen(to64(q), to64(k), to64(v), to64(sink), cu.numpy(), W)
    out, lse = swa.swa_sink_prefill_varlen(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu),
                                           cu.to(gpu), max(lens), W)
    torch.cuda.synchronize()
    check_out(out, ref_out, BF16)
    check_lse(lse, ref_lse, BF16)


@pytest.mark.parametrize("i,B,Sq,Skv,Hq,Hkv,D", _cases("global", 12, 1003))
def test_global_sweep(gpu, i, B, Sq, Skv, Hq, Hkv, D):
    q, k, v, sink = inputs.attention_inputs(303, i, B, Sq, Skv, Hq, Hkv, D, BF16)
    ref_out, ref_lse = oracle.global_attn(to64(q), to64(k), to64(v), to64(sink))
    args = (q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu))
    for fn in (swa.global_sink_attn, swa.global_sink_attn_noalloc):
        out, lse = fn(*args)
        torch.cuda.synchronize()
        check_out(out, ref_out, BF16)
        check_lse(lse, ref_lse, BF16)


@pytest.mark.parametrize("i,B,T,Hq,Hkv,D,W,R", _cases("ring", 12, 1004))
def test_ring_decode_sweep(gpu, i, B, T, Hq, Hkv, D, W, R):
    q, kc, vc, sink = inputs.ring_inputs(304, i, B, T, Hq, Hkv, R, D, BF16)
    lens = inputs.cache_lengths(B, T, 3 * R, 304 + i)
    ref_out, ref_lse = oracle.ring_decode(to64(q), to64(kc), to64(vc), to64(sink), lens.numpy(),
                                          window=W)
    out, lse = swa.swa_sink_decode_ring(q.to(gpu), kc.to(gpu), vc.to(gpu), sink.to(gpu), W,
                                        lens.to(gpu))
    torch.cuda.synchronize()
    check_out(out, ref_out, BF16)
    check_lse(lse, ref_lse.transpose(0, 2, 1), BF16)


@pytest.mark.parametrize("i,B,S,Hq,Hkv,D,W", _cases("backward", 10, 1005))
def test_backward_sweep(gpu, i, B, S, Hq, Hkv, D, W):
    q, k, v, sink = inputs.attention_inputs(305, i, B, S, S, Hq, Hkv, D, BF16)
    g = inputs.upstream_grad(305, i, B, S, Hq, D, BF16)
    qd, kd, vd, sd, gd = (t.to(gpu) for t in (q, k, v, sink, g))
    if W >= S:
        out, lse = swa.global_sink_attn(qd, kd, vd, sd)
    else:
        out, lse = swa.swa_sink_prefill(qd, kd, vd, sd, W)
    got = swa.swa_sink_backward(qd, kd, vd, sd, out, lse, gd, W)
    torch.cuda.synchronize()
    args = (to64(q), to64(k), to64(v), to64(sink), to64(g), W)
    ref = oracle.attend_backward(*args)
    model = rounded_backward(*args)
    for n, (name, a, r) in enumerate(zip(("dq", "dk", "dv", "dsink"), got, ref)):
        c = None if name == "dsink" else max(GRAD_C[BF16], 1.25 * scaled_error(model[n], r))
        check_grad(a, r, BF16, name, c=c)
