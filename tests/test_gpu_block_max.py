"""GPU parity: global_sink_attn_block_max against the fp64 oracle, through
the C ABI: the block maxima of the scaled logits, and out / lse unchanged
(bit-identical to global_sink_attn)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.parity import to64

pytestmark = pytest.mark.gpu

# Logits are fp32 sums of exact bf16 products; the oracle sums in fp64.
BMAX_ATOL, BMAX_RTOL = 1e-4, 1e-5


def check_bmax(gpu, ref):
    g = to64(gpu)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), "visible-block pattern differs"
    fin = np.isfinite(ref)
    assert np.isfinite(g[fin]).all()
    err = np.abs(g[fin] - ref[fin])
    bad = err > BMAX_ATOL + BMAX_RTOL * np.abs(ref[fin])
    assert not bad.any(), "%d block maxima off (worst %.3g)" % (int(bad.sum()), float(err.max()))


CASES = [
    # B, S_q, S_kv, Hq, Hkv, D, block_k
    (1, 300, 300, 8, 1, 128, 128),
    (2, 257, 257, 8, 2, 64, 32),
    (1, 100, 1000, 16, 2, 128, 96),
    (2, 5, 700, 8, 1, 128, 64),
    (1, 1000, 1000, 64, 8, 128, 128),
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,bk", CASES)
def test_block_max_matches_oracle(gpu, B, Sq, Skv, Hq, Hkv, D, bk):
    q, k, v, sink = inputs.attention_inputs(93, 0, B, Sq, Skv, Hq, Hkv, D, torch.bfloat16, "cuda")
    out, lse, bm = swa.global_sink_attn_block_max(q, k, v, sink, block_k=bk)
    torch.cuda.synchronize()
    check_bmax(bm, oracle.block_max(to64(q), to64(k), bk))
    # out and lse are exactly those of global_sink_attn on the streaming path
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    if Hq // Hkv * Sq > 64:
        swa.global_sink_attn(q, k, v, sink, out=out2, lse=lse2)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_block_max_overwrites_every_element(gpu):
    B, S, Hq, Hkv, D, bk = 1, 200, 8, 1, 128, 64
    q, k, v, sink = inputs.attention_inputs(94, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    bm = torch.full((B, Hq, 7, 4), float("nan"), device="cuda")
    swa.global_sink_attn_block_max(q, k, v, sink, block_k=bk, block_max=bm)
    torch.cuda.synchronize()
    check_bmax(bm, oracle.block_max(to64(q), to64(k), bk))


def test_block_max_full_size_sampled(gpu):
    """The global layer of the hybrid stack (B=1, S=65536, Hq=64, Hkv=8,
    D=128), block_k 128: sampled (head, 32-row block) rows of the output,
    each checked over all 512 key blocks against the oracle on those rows."""
    B, S, Hq, Hkv, D, bk = 1, 65536, 64, 8, 128, 128
    q, k, v, sink = inputs.attention_inputs(4, 5, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    _, _, bm = swa.global_sink_attn_block_max(q, k, v, sink, block_k=bk, want_lse=False)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for h, qb in [(0, 0), (13, 1000), (63, 2047)]:
        r0, r1 = 32 * qb, min(S, 32 * qb + 32)
        g = h // G
        qs = to64(q[:, r0:r1, h:h + 1])
        ks = to64(k[:, :r1, g:g + 1])                 # keys up to the block's last row
        ref = oracle.block_max(qs, ks, bk)[0, 0, 0]     # [ceil(r1 / bk)]
        full = np.full(S // bk, -np.inf)
        full[:ref.shape[0]] = ref
        check_bmax(bm[0, h, qb], full)
