"""global_sink_attn_noalloc (the entry point that allocates nothing: split
partials in the library's static per-GPU scratch array) against
global_sink_attn (same kernels, caller workspace), through the C ABI.

Two scratch-using calls in a row, the second with a smaller input (the array
keeps the first call's contents), each compared element by element with the
workspace entry point, and once with the fp64 oracle; then a prefill-shaped
call, which takes the streaming kernel and no scratch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


@pytest.mark.parametrize("B,Sq,Skv", [(8, 1, 65536), (2, 3, 5000), (1, 200, 200)])
def test_noalloc_equals_workspace_entry_point(gpu, B, Sq, Skv):
    Hq, Hkv, D = 64, 8, 128
    print("noalloc case", B, Sq, Skv, flush=True)
    q, k, v, sink = inputs.attention_inputs(140, Sq, B, Sq, Skv, Hq, Hkv, D, BF16, gpu)
    needs_scratch = swa.global_sink_attn_workspace_bytes(B, Hq, Hkv, Sq, Skv, D) > 0
    assert needs_scratch == (Sq < 200)
    ref_out, ref_lse = swa.global_sink_attn(q, k, v, sink)
    out, lse = swa.global_sink_attn_noalloc(q, k, v, sink)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    # the last sequence against the oracle (all heads, all rows)
    b = B - 1
    o64, l64 = oracle.global_attn(to64(q[b:b + 1]), to64(k[b:b + 1]), to64(v[b:b + 1]),
                                  to64(sink))
    check_out(out[b:b + 1], o64, BF16)
    check_lse(lse[b:b + 1], l64, BF16)


def test_noalloc_repeated_calls_shrinking(gpu):
    """Back-to-back calls on one stream with shrinking sizes: each result
    equals the workspace entry point's."""
    Hq, Hkv, D = 16, 2, 128
    for B, Sq, Skv in [(4, 4, 9000), (3, 2, 3000), (1, 1, 33)]:
        q, k, v, sink = inputs.attention_inputs(141, Sq, B, Sq, Skv, Hq, Hkv, D, BF16, gpu)
        a = swa.global_sink_attn_noalloc(q, k, v, sink)
        r = swa.global_sink_attn(q, k, v, sink)
        torch.cuda.synchronize()
        assert torch.equal(a[0], r[0]) and torch.equal(a[1], r[1])
