"""GPU parity: global_sink_attn (prefill-shaped, streaming kernel) and wide-window
swa_sink_prefill against the fp64 oracle, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def global_case(gpu, cfg, B, Sq, Skv, Hq, Hkv, D, dtype, sink_override=None):
    q, k, v, sink = inputs.attention_inputs(cfg, 0, B, Sq, Skv, Hq, Hkv, D, dtype)
    if sink_override is not None:
        sink = torch.full((Hq,), float(sink_override))
    ref_out, ref_lse = oracle.global_attn(to64(q), to64(k), to64(v), to64(sink))
    out, lse = swa.global_sink_attn(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu))
    torch.cuda.synchronize()
    check_out(out, ref_out, dtype)
    check_lse(lse, ref_lse, dtype)


GLOBAL_CASES = [
    # B, Sq, Skv, Hq, Hkv, D
    (1, 512, 512, 8, 1, 128),
    (2, 333, 333, 64, 8, 128),
    (1, 1000, 1000, 16, 2, 64),
    (1, 65, 700, 8, 1, 128),        # queries at the end of a longer key sequence
    (2, 40, 41, 16, 1, 128),        # G = 16: each wave serves two heads
    (1, 1, 1, 1, 1, 128),
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D", GLOBAL_CASES)
def test_global_prefill_bf16(gpu, B, Sq, Skv, Hq, Hkv, D):
    global_case(gpu, 110, B, Sq, Skv, Hq, Hkv, D, torch.bfloat16)


def test_global_prefill_sink_neg_inf(gpu):
    global_case(gpu, 111, 1, 300, 300, 8, 1, 128, torch.bfloat16, -np.inf)


def test_global_prefill_f32(gpu):
    global_case(gpu, 112, 1, 200, 260, 8, 2, 128, torch.float32)


@pytest.mark.parametrize("W", [130, 200, 511, 4096])
def test_wide_window_prefill(gpu, W):
    B, S, Hq, Hkv, D = 1, 900, 16, 2, 128
    q, k, v, sink = inputs.attention_inputs(113, 0, B, S, S, Hq, Hkv, D, torch.bfloat16)
    ref_out, ref_lse = oracle.swa_prefill(to64(q), to64(k), to64(v), to64(sink), W)
    out, lse = swa.swa_sink_prefill(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu), W)
    torch.cuda.synchronize()
    check_out(out, ref_out, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)


def test_window_ge_S_equals_global(gpu):
    """swa_sink_prefill with window >= S is the global layer (two different kernels)."""
    B, S, Hq, Hkv, D = 1, 700, 64, 8, 128
    q, k, v, sink = inputs.attention_inputs(114, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    o1, l1 = swa.swa_sink_prefill(q, k, v, sink, S)
    o2, l2 = swa.global_sink_attn(q, k, v, sink)
    torch.cuda.synchronize()
    assert (o1.double() - o2.double()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_global_64k_sampled_rows(gpu):
    """The global layer of the hybrid 5:1 stack at full size (S=65536, Hq=64,
    Hkv=8, D=128), checked on 608 rows: the first and last 32, and one seeded
    random row in every fourth 32-row query block (512 blocks spread over the
    whole sequence, so every stage of the longest-first launch order is
    sampled)."""
    B, S, Hq, Hkv, D = 1, 65536, 64, 8, 128
    q, k, v, sink = inputs.attention_inputs(4, 5, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    out, lse = swa.global_sink_attn(q, k, v, sink)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    blocks = np.arange(0, S // 32, 4)
    rows = np.array(sorted(set(range(32)) | set(range(S - 32, S)) |
                           set((32 * blocks + rng.integers(0, 32, len(blocks))).tolist())))
    assert len(rows) >= 512
    idx = torch.as_tensor(rows, device=gpu)
    ref_out, ref_lse = oracle.global_rows(to64(q[0].index_select(0, idx)), np.zeros(len(rows)),
                                          rows, to64(k), to64(v), to64(sink))
    check_out(out[0].index_select(0, idx), ref_out, torch.bfloat16)
    check_lse(lse[0].index_select(1, idx).T, ref_lse, torch.bfloat16)


def test_global_64k_real_token_mass_identity(gpu):
    B, S, Hq, Hkv, D = 1, 65536, 64, 8, 128
    q, k, _, sink = inputs.attention_inputs(4, 5, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    v = torch.ones_like(k)
    out, lse = swa.global_sink_attn(q, k, v, sink)
    torch.cuda.synchronize()
    mass = 1.0 - torch.exp(sink.double()[None, :, None] - lse.double())
    expect = mass.permute(0, 2, 1)[..., None].expand(B, S, Hq, D)
    err = (out.double() - expect).abs()
    assert bool((err <= 2e-2 + 1e-2 * expect.abs()).all()), float(err.max())


def test_stream_repeat_runs_bit_identical(gpu):
    """Repeated runs of the streaming kernel (global causal layer, and a wide
    window) on the same inputs are bit-identical and finite."""
    q, k, v, sink = inputs.attention_inputs(96, 0, 1, 4096, 4096, 64, 8, 128, torch.bfloat16, "cuda")
    o1, l1 = swa.global_sink_attn(q, k, v, sink)
    w1, wl1 = swa.swa_sink_prefill(q, k, v, sink, 1000)
    assert bool(torch.isfinite(o1).all()) and bool(torch.isfinite(w1).all())
    for _ in range(6):
        o2, l2 = swa.global_sink_attn(q, k, v, sink)
        w2, wl2 = swa.swa_sink_prefill(q, k, v, sink, 1000)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert torch.equal(w1, w2) and torch.equal(wl1, wl2)
