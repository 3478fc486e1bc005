"""GPU parity at the long-context sizes: the 262144-token window-128 prefill
(its chunk buffer windows near the 31-bit range limit) on sampled rows, and
the global decode of 8 sequences over 262144 keys (split-KV partials plus
combine) on one full sequence, and the streaming kernel past 32-bit key
offsets, against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.parity import check_lse, check_out, to64
from tests.test_gpu_block_max import check_bmax

pytestmark = pytest.mark.gpu

S_LONG = 262144


def test_swa_prefill_262144_sampled_rows(gpu):
    """First and last 256 rows, 2048 seeded random rows, all 64 heads."""
    B, Hq, Hkv, D, W = 1, 64, 8, 128, 128
    print("prefill 262144", flush=True)
    q, k, v, sink = inputs.attention_inputs(5, 0, B, S_LONG, S_LONG, Hq, Hkv, D, torch.bfloat16,
                                            gpu)
    out, lse = swa.swa_sink_prefill(q, k, v, sink, W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5001)
    rows = np.array(sorted(set(range(256)) | set(range(S_LONG - 256, S_LONG))
                           | set(rng.integers(0, S_LONG, 2048).tolist())))
    idx = torch.as_tensor(rows, device=gpu)
    ref_out, ref_lse = oracle.swa_prefill_rows(to64(q[0].index_select(0, idx)),
                                               np.zeros(len(rows)), rows, to64(k), to64(v),
                                               to64(sink), W)
    check_out(out[0].index_select(0, idx), ref_out, torch.bfloat16)
    check_lse(lse[0].index_select(1, idx).T, ref_lse, torch.bfloat16)


def test_swa_prefill_65536_chunk_boundaries(gpu):
    """The sliding-window layer of the hybrid 5:1 stack at full size
    (S=65536, Hq=64, Hkv=8, D=128, window 128) in the launch the benchmark
    times: the prefill then runs 2048-position chunks, each starting with its
    own 127-key halo.  Rows around every chunk boundary (c-1, c, c+1, c+31,
    c+32, c+126, c+127, c+128), the first and last 128 rows and 1024 seeded
    random rows, all 64 heads."""
    B, S, Hq, Hkv, D, W = 1, 65536, 64, 8, 128, 128
    print("prefill 65536", flush=True)
    q, k, v, sink = inputs.attention_inputs(4, 1, B, S, S, Hq, Hkv, D, torch.bfloat16, gpu)
    out, lse = swa.swa_sink_prefill(q, k, v, sink, W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4001)
    edge = {c + d for c in range(0, S, 2048) for d in (-1, 0, 1, 31, 32, 126, 127, 128)}
    rows = np.array(sorted({r for r in edge if 0 <= r < S} | set(range(128))
                           | set(range(S - 128, S)) | set(rng.integers(0, S, 1024).tolist())))
    idx = torch.as_tensor(rows, device=gpu)
    ref_out, ref_lse = oracle.swa_prefill_rows(to64(q[0].index_select(0, idx)),
                                               np.zeros(len(rows)), rows, to64(k), to64(v),
                                               to64(sink), W)
    check_out(out[0].index_select(0, idx), ref_out, torch.bfloat16)
    check_lse(lse[0].index_select(1, idx).T, ref_lse, torch.bfloat16)


@pytest.mark.parametrize("seq", [0, 7])
def test_global_decode_262144_one_sequence(gpu, seq):
    """One of the 8 sequences in full (all 64 heads), as the bench launches it."""
    B, Hq, Hkv, D = 8, 64, 8, 128
    print("global decode 262144, sequence", seq, flush=True)
    q, k, v, sink = inputs.attention_inputs(5, 1, B, 1, S_LONG, Hq, Hkv, D, torch.bfloat16, gpu)
    out, lse = swa.global_sink_attn(q, k, v, sink)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.global_rows(to64(q[seq]), np.zeros(1), np.array([S_LONG - 1]),
                                          to64(k[seq:seq + 1]), to64(v[seq:seq + 1]), to64(sink))
    check_out(out[seq], ref_out, torch.bfloat16)
    check_lse(lse[seq].T, ref_lse, torch.bfloat16)


def test_stream_kernel_keys_past_32bit_offsets(gpu):
    """Keys whose byte offsets within one KV head's column pass 2^32 (2^21 + 37
    positions of 8 KV heads x 128 dims): the streaming kernel then builds its
    copy descriptors per tile.  All 69 query rows (3 blocks, ragged) of the
    two query heads of KV head 0, with their block maxima."""
    B, Hq, Hkv, D, S_q, bk = 1, 16, 8, 128, 69, 128
    S_kv = (1 << 21) + 37
    assert (S_kv + 32) * Hkv * D * 2 > (1 << 32)
    print("block-max global over", S_kv, "keys", flush=True)
    q, k, v, sink = inputs.attention_inputs(5, 2, B, S_q, S_kv, Hq, Hkv, D, torch.bfloat16, gpu)
    out, lse, bm = swa.global_sink_attn_block_max(q, k, v, sink, block_k=bk)
    torch.cuda.synchronize()
    k0, v0 = to64(k[:, :, 0:1]), to64(v[:, :, 0:1])
    del k, v
    rows = np.arange(S_kv - S_q, S_kv)
    ref_out, ref_lse = oracle.global_rows(to64(q[0, :, 0:2]), np.zeros(S_q), rows, k0, v0,
                                          to64(sink[0:2]))
    check_out(out[0, :, 0:2], ref_out, torch.bfloat16)
    check_lse(lse[0, 0:2].T, ref_lse, torch.bfloat16)
    check_bmax(bm[:, 0:2], oracle.block_max(to64(q[:, :, 0:2]), k0, bk))
