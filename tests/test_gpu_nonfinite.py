"""GPU parity with non-finite data, through the C ABI, against the fp64 oracle.

* Partly filled rings (L < ring slots): the slots no token has reached hold
  whatever bits the cache was allocated with.  Here they hold bf16 NaN and
  Inf patterns; the oracle never reads them, and the kernels must not let
  them reach a result either.
* NaN in one query row, one key row or one head's sink propagates to exactly
  the outputs the definition makes NaN (the oracle's pattern), and leaves
  every other output unchanged.
* NaN in one value row: every output that sees the row is NaN; besides, the
  matrix products may spread it to rows of the same 32-key tile that do not
  see it (their weight for it is 0, and 0 * NaN = NaN) -- nowhere else.

Sources: the sink term of the technical-report digest, 前置知识 / 注意力sink偏置;
the fixed-size sliding-window cache of the pwwt.cn article, §1.1.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.parity import (check_lse, check_lse_nonfinite, check_out, check_out_nonfinite,
                          to64)

pytestmark = pytest.mark.gpu

# bf16 bit patterns: quiet NaN, +Inf, -Inf, a NaN with payload, negative NaN
BAD_BITS = [0x7FC0, 0x7F80, 0xFF80, 0x7F81, 0xFFC1]


def bf16_bits(bits: int) -> torch.Tensor:
    return torch.tensor([bits], dtype=torch.int32).to(torch.int16).view(torch.bfloat16)[0]


def poison_unwritten(cache: torch.Tensor, lens, salt: int) -> torch.Tensor:
    """cache [B, Hkv, R, D] with slots L_b .. R-1 of sequence b (L_b < R, no
    wrap yet) filled with non-finite bf16 patterns."""
    c = cache.clone()
    R = c.shape[2]
    for b, L in enumerate(lens):
        if L < R:
            c[b, :, max(L, 0):] = bf16_bits(BAD_BITS[(b + salt) % len(BAD_BITS)])
    return c


@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("ring_extra", [0, 3])
def test_partly_filled_ring_ignores_unwritten_slots(gpu, T, ring_extra):
    """Rings with L in {1, 3, 77, 127} tokens (T_q = 1 and 4; L < T_q leaves
    the first drafts without keys), unwritten slots holding NaN/Inf bits;
    swa_sink_decode (ring = window = 128) and swa_sink_decode_ring (131-slot
    rollback ring, window 128)."""
    B, Hq, Hkv, D, W = 4, 64, 8, 128, 128
    R = W + ring_extra
    lens = [1, 3, 77, 127]
    q, kc, vc, sink = inputs.ring_inputs(120, ring_extra, B, T, Hq, Hkv, R, D, torch.bfloat16)
    kc, vc = poison_unwritten(kc, lens, 0), poison_unwritten(vc, lens, 2)
    cl = torch.tensor(lens, dtype=torch.int32)
    ref_out, ref_lse = oracle.ring_decode(to64(q), to64(kc), to64(vc), to64(sink), cl.numpy(), W)
    if ring_extra == 0:
        out, lse = swa.swa_sink_decode(q.to(gpu), kc.to(gpu), vc.to(gpu), sink.to(gpu), cl.to(gpu))
    else:
        out, lse = swa.swa_sink_decode_ring(q.to(gpu), kc.to(gpu), vc.to(gpu), sink.to(gpu), W,
                                            cl.to(gpu))
    torch.cuda.synchronize()
    check_out(out, ref_out, torch.bfloat16)
    check_lse(lse, ref_lse.transpose(0, 2, 1), torch.bfloat16)


def test_partly_filled_ring_f32(gpu):
    """The float32 path reads only the visible positions; same check."""
    B, T, Hq, Hkv, D, W = 4, 4, 8, 2, 64, 128
    lens = [1, 3, 77, 127]
    q, kc, vc, sink = inputs.ring_inputs(121, 0, B, T, Hq, Hkv, W, D, torch.float32)
    for b, L in enumerate(lens):
        kc[b, :, L:] = float("nan")
        vc[b, :, L:] = float("inf")
    cl = torch.tensor(lens, dtype=torch.int32)
    ref_out, ref_lse = oracle.ring_decode(to64(q), to64(kc), to64(vc), to64(sink), cl.numpy())
    out, lse = swa.swa_sink_decode(q.to(gpu), kc.to(gpu), vc.to(gpu), sink.to(gpu), cl.to(gpu))
    torch.cuda.synchronize()
    check_out(out, ref_out, torch.float32)
    check_lse(lse, ref_lse.transpose(0, 2, 1), torch.float32)


# --- NaN in q, k or the sink: exactly the oracle's NaN pattern ----------------

def plant(q, k, v, sink, what, qi, kj):
    """NaN in query row qi (head 1), key row kj (KV head 0) or value row kj
    (KV head 0) of sequence 0, or in the sink of head 2."""
    q, k, v, sink = q.clone(), k.clone(), v.clone(), sink.clone()
    if what == "q":
        q[0, qi, 1] = float("nan")
    elif what == "k":
        k[0, kj, 0] = float("nan")
    elif what == "v":
        v[0, kj, 0] = float("nan")
    else:
        sink[2] = float("nan")
    return q, k, v, sink


PREFILL_NAN_CASES = [
    # what, S, Hq, Hkv, W  (W 128 / 98: ring kernel; 511 and global: streaming kernel)
    ("q", 300, 16, 2, 128), ("k", 300, 16, 2, 128), ("sink", 300, 16, 2, 128),
    ("q", 300, 16, 2, 98), ("k", 300, 16, 2, 98),
    ("q", 700, 16, 2, 511), ("k", 700, 16, 2, 511), ("sink", 700, 16, 2, 511),
    ("q", 260, 8, 1, 0), ("k", 260, 8, 1, 0), ("sink", 260, 8, 1, 0),
]


@pytest.mark.parametrize("what,S,Hq,Hkv,W", PREFILL_NAN_CASES)
def test_prefill_nan_pattern(gpu, what, S, Hq, Hkv, W):
    """W = 0 means the global layer (global_sink_attn)."""
    D = 128
    q, k, v, sink = inputs.attention_inputs(122, 0, 2, S, S, Hq, Hkv, D, torch.bfloat16)
    q, k, v, sink = plant(q, k, v, sink, what, qi=S // 2 + 3, kj=S // 3 + 5)
    if W == 0:
        ref_out, ref_lse = oracle.global_attn(to64(q), to64(k), to64(v), to64(sink))
        out, lse = swa.global_sink_attn(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu))
    else:
        ref_out, ref_lse = oracle.swa_prefill(to64(q), to64(k), to64(v), to64(sink), W)
        out, lse = swa.swa_sink_prefill(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu), W)
    torch.cuda.synchronize()
    assert np.isnan(ref_out).any() and np.isnan(ref_lse).any()
    check_out_nonfinite(out, ref_out, torch.bfloat16)
    check_lse_nonfinite(lse, ref_lse, torch.bfloat16)


@pytest.mark.parametrize("what", ["q", "k", "sink"])
@pytest.mark.parametrize("T", [1, 4])
def test_ring_decode_nan_pattern(gpu, what, T):
    """Full and partly filled rings; the NaN key sits at a slot that the
    earlier drafts of a T_q = 4 step do not see (they must stay finite)."""
    B, Hq, Hkv, D, W = 2, 16, 2, 128, 128
    q, kc, vc, sink = inputs.ring_inputs(123, T, B, T, Hq, Hkv, W, D, torch.bfloat16)
    lens = [1000, 90]
    # sequence 0: newest position 999 is in slot 999 % 128 = 103
    q, kc, vc, sink = plant(q, kc.transpose(1, 2), vc.transpose(1, 2), sink, what,
                            qi=T - 1, kj=999 % W)
    kc, vc = kc.transpose(1, 2).contiguous(), vc.transpose(1, 2).contiguous()
    cl = torch.tensor(lens, dtype=torch.int32)
    ref_out, ref_lse = oracle.ring_decode(to64(q), to64(kc), to64(vc), to64(sink), cl.numpy())
    out, lse = swa.swa_sink_decode(q.to(gpu), kc.to(gpu), vc.to(gpu), sink.to(gpu), cl.to(gpu))
    torch.cuda.synchronize()
    assert np.isnan(ref_out).any()
    if what == "k" and T == 4:
        assert not np.isnan(ref_out[0, :T - 1]).any()      # earlier drafts do not see it
    check_out_nonfinite(out, ref_out, torch.bfloat16)
    check_lse_nonfinite(lse, ref_lse.transpose(0, 2, 1), torch.bfloat16)


@pytest.mark.parametrize("what", ["q", "k", "sink"])
def test_split_kv_nan_pattern(gpu, what):
    """Global decode (split-KV partials, combine adds the sink once)."""
    B, Sq, Skv, Hq, Hkv, D = 2, 2, 5000, 16, 2, 128
    q, k, v, sink = inputs.attention_inputs(124, 0, B, Sq, Skv, Hq, Hkv, D, torch.bfloat16)
    q, k, v, sink = plant(q, k, v, sink, what, qi=1, kj=4321)
    ref_out, ref_lse = oracle.global_attn(to64(q), to64(k), to64(v), to64(sink))
    out, lse = swa.global_sink_attn(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu))
    torch.cuda.synchronize()
    assert np.isnan(ref_out).any()
    check_out_nonfinite(out, ref_out, torch.bfloat16)
    check_lse_nonfinite(lse, ref_lse, torch.bfloat16)


def test_nan_sink_without_visible_keys(gpu):
    """A row with no visible key (L < T_q) keeps out = 0 under a NaN sink; its
    lse (= the sink) is NaN."""
    B, T, Hq, Hkv, D, W = 1, 4, 8, 1, 128, 128
    q, kc, vc, sink = inputs.ring_inputs(125, 0, B, T, Hq, Hkv, W, D, torch.bfloat16)
    sink[3] = float("nan")
    cl = torch.tensor([2], dtype=torch.int32)
    ref_out, ref_lse = oracle.ring_decode(to64(q), to64(kc), to64(vc), to64(sink), cl.numpy())
    out, lse = swa.swa_sink_decode(q.to(gpu), kc.to(gpu), vc.to(gpu), sink.to(gpu), cl.to(gpu))
    torch.cuda.synchronize()
    assert (ref_out[0, :2] == 0).all() and np.isnan(ref_lse[0, 0, 3])
    check_out_nonfinite(out, ref_out, torch.bfloat16)
    check_lse_nonfinite(lse, ref_lse.transpose(0, 2, 1), torch.bfloat16)


@pytest.mark.parametrize("W", [128, 0])
def test_prefill_nan_value_row(gpu, W):
    """NaN in one value row: the rows that see it are NaN (as in the oracle);
    the GPU may also turn rows NaN whose key tiles include the row's tile,
    and no others.  W = 0: the global layer."""
    S, Hq, Hkv, D = 400, 16, 2, 128
    kj = 201
    q, k, v, sink = inputs.attention_inputs(126, 0, 1, S, S, Hq, Hkv, D, torch.bfloat16)
    q, k, v, sink = plant(q, k, v, sink, "v", 0, kj)
    if W == 0:
        ref_out, ref_lse = oracle.global_attn(to64(q), to64(k), to64(v), to64(sink))
        out, lse = swa.global_sink_attn(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu))
        lo_t = np.zeros(S, dtype=np.int64)
    else:
        ref_out, ref_lse = oracle.swa_prefill(to64(q), to64(k), to64(v), to64(sink), W)
        out, lse = swa.swa_sink_prefill(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu), W)
        # the tiles a row's 32-row step reads: from the oldest key of its first row
        lo_t = np.maximum(0, (np.arange(S) // 32) * 32 - W + 1) // 32
    torch.cuda.synchronize()
    hi_t = (np.minimum(S - 1, (np.arange(S) // 32) * 32 + 31)) // 32
    shares = (lo_t <= kj // 32) & (kj // 32 <= hi_t)            # [S]
    spread = np.zeros(ref_out.shape, bool)
    spread[0, shares, 0:Hq // Hkv, :] = True                    # heads of KV head 0
    check_out_nonfinite(out, ref_out, torch.bfloat16, may_spread=spread)
    check_lse(lse, ref_lse, torch.bfloat16)
