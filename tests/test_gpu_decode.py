"""GPU parity: swa_sink_decode (ring cache) and decode-shaped global_sink_attn
(split-KV + combine) against the fp64 oracle, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def ring_case(gpu, cfg, B, T, Hq, Hkv, W, D, dtype, lens=None, sink_override=None):
    q, kc, vc, sink = inputs.ring_inputs(cfg, 0, B, T, Hq, Hkv, W, D, dtype)
    if sink_override is not None:
        sink = torch.full((Hq,), float(sink_override))
    cl = None if lens is None else torch.as_tensor(lens, dtype=torch.int32)
    ref_out, ref_lse = oracle.ring_decode(to64(q), to64(kc), to64(vc), to64(sink),
                                          None if cl is None else cl.numpy())
    out, lse = swa.swa_sink_decode(q.to(gpu), kc.to(gpu), vc.to(gpu), sink.to(gpu),
                                   None if cl is None else cl.to(gpu))
    torch.cuda.synchronize()
    check_out(out, ref_out, dtype)
    check_lse(lse, ref_lse.transpose(0, 2, 1), dtype)


RING_CASES = [
    # B, T, Hq, Hkv, W, D, lens (None = full rings)
    (3, 1, 8, 1, 128, 128, None),
    (3, 4, 8, 1, 128, 128, None),
    (4, 1, 64, 8, 128, 128, [128, 129, 5000, 1000001]),
    (4, 4, 64, 8, 128, 128, [4, 77, 131, 9999]),
    (2, 2, 16, 2, 16, 64, [16, 40]),
    (2, 3, 6, 2, 100, 128, [100, 250]),
    (2, 1, 8, 8, 200, 128, [150, 431]),
    (2, 4, 32, 2, 128, 64, [64, 300]),          # G*T = 64: two column tiles
    (1, 4, 8, 1, 128, 128, [2]),                # L < T: two rows see no key
]


@pytest.mark.parametrize("B,T,Hq,Hkv,W,D,lens", RING_CASES)
def test_ring_decode_bf16(gpu, B, T, Hq, Hkv, W, D, lens):
    ring_case(gpu, 95, B, T, Hq, Hkv, W, D, torch.bfloat16, lens)


@pytest.mark.parametrize("T", [1, 4])
def test_ring_decode_f32(gpu, T):
    ring_case(gpu, 96, 3, T, 8, 2, 128, 64, torch.float32, [128, 300, 7])


def test_ring_decode_sink_neg_inf(gpu):
    ring_case(gpu, 97, 2, 4, 8, 1, 128, 128, torch.bfloat16, [130, 260], -np.inf)


@pytest.mark.parametrize("T", [1, 4])
def test_ring_decode_full_workload(gpu, T):
    """Batched decode workload at full size: B=256, Hq=64, Hkv=8, D=128, 128-slot rings."""
    ring_case(gpu, 3, 256, T, 64, 8, 128, 128, torch.bfloat16)


def test_ring_decode_matches_prefill_last_row(gpu):
    """Filling the ring from a sequence (slot = position mod W) and decoding
    its last token reproduces the prefill's last row."""
    B, S, Hq, Hkv, D, W = 2, 300, 8, 1, 128, 128
    q, k, v, sink = inputs.attention_inputs(98, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    pre, pre_lse = swa.swa_sink_prefill(q, k, v, sink, W)
    pos = torch.arange(S - W, S, device=gpu)
    kc = torch.empty(B, Hkv, W, D, dtype=k.dtype, device=gpu)
    vc = torch.empty_like(kc)
    kc[:, :, pos % W] = k[:, pos].permute(0, 2, 1, 3)
    vc[:, :, pos % W] = v[:, pos].permute(0, 2, 1, 3)
    lens = torch.full((B,), S, dtype=torch.int32, device=gpu)
    dec, dec_lse = swa.swa_sink_decode(q[:, -1:].contiguous(), kc, vc, sink, lens)
    torch.cuda.synchronize()
    err = (dec[:, 0].double() - pre[:, -1].double()).abs().max().item()
    assert err <= 2e-2, err
    assert (dec_lse[:, :, 0] - pre_lse[:, :, -1]).abs().max().item() <= 1e-3


# --- global attention, decode-shaped (split over the keys, sink added once) -----

def global_case(gpu, cfg, B, Sq, Skv, Hq, Hkv, D, dtype, device="cpu"):
    q, k, v, sink = inputs.attention_inputs(cfg, 0, B, Sq, Skv, Hq, Hkv, D, dtype, device)
    ref_out, ref_lse = oracle.global_attn(to64(q), to64(k), to64(v), to64(sink))
    out, lse = swa.global_sink_attn(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu))
    torch.cuda.synchronize()
    check_out(out, ref_out, dtype)
    check_lse(lse, ref_lse, dtype)


GLOBAL_DECODE_CASES = [
    (2, 1, 1000, 64, 8, 128),
    (2, 4, 1000, 64, 8, 128),
    (3, 3, 4097, 16, 2, 64),
    (1, 1, 1, 8, 1, 128),
    (1, 2, 130, 8, 8, 128),
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D", GLOBAL_DECODE_CASES)
def test_global_decode_bf16(gpu, B, Sq, Skv, Hq, Hkv, D):
    global_case(gpu, 99, B, Sq, Skv, Hq, Hkv, D, torch.bfloat16)


def test_global_decode_f32(gpu):
    global_case(gpu, 100, 2, 2, 777, 8, 2, 64, torch.float32)


def test_global_decode_long_cache(gpu):
    """Long-context global decode: 65536-token cache, B=2, Hq=64, Hkv=8, D=128."""
    global_case(gpu, 5, 2, 1, 65536, 64, 8, 128, torch.bfloat16, "cuda")


def test_split_count_does_not_change_result(gpu):
    """The split plan depends on the batch size; rows of a sequence decoded
    alone and inside a batch must agree (the sink is added once either way)."""
    q, k, v, sink = inputs.attention_inputs(101, 0, 4, 1, 20000, 64, 8, 128, torch.bfloat16, "cuda")
    full, full_lse = swa.global_sink_attn(q, k, v, sink)
    one, one_lse = swa.global_sink_attn(q[:1].contiguous(), k[:1].contiguous(),
                                        v[:1].contiguous(), sink)
    torch.cuda.synchronize()
    assert (full[:1].double() - one.double()).abs().max().item() <= 1e-2
    assert (full_lse[:1] - one_lse).abs().max().item() <= 1e-4


def test_global_decode_256k_full_size(gpu):
    """Long-context global decode at full size and in the launch configuration
    the benchmark times: B=8, one query token, 262144 cached keys, Hq=64,
    Hkv=8, D=128.  Two sequences are compared with the oracle; the V == 1
    identity out = 1 - exp(s_h - lse) is checked on all eight."""
    B, Sq, Skv, Hq, Hkv, D = 8, 1, 262144, 64, 8, 128
    q, k, v, sink = inputs.attention_inputs(5, 1, B, Sq, Skv, Hq, Hkv, D, torch.bfloat16, "cuda")
    out, lse = swa.global_sink_attn(q, k, v, sink)
    torch.cuda.synchronize()
    for b in (0, 5):
        ref_out, ref_lse = oracle.global_attn(to64(q[b:b + 1]), to64(k[b:b + 1]), to64(v[b:b + 1]),
                                              to64(sink))
        check_out(out[b:b + 1], ref_out, torch.bfloat16)
        check_lse(lse[b:b + 1], ref_lse, torch.bfloat16)
    ones = torch.ones_like(v)
    del v
    out1, lse1 = swa.global_sink_attn(q, k, ones, sink)
    torch.cuda.synchronize()
    mass = 1.0 - torch.exp(sink.double()[None, :, None] - lse1.double())      # B Hq Sq
    expect = mass.permute(0, 2, 1)[..., None].expand(B, Sq, Hq, D)
    err = (out1.double() - expect).abs()
    assert bool((err <= 2e-2 + 1e-2 * expect.abs()).all()), float(err.max())
