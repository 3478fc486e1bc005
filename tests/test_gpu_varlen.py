"""GPU parity: swa_sink_prefill_varlen (HIP, through the C ABI) against the
fp64 oracle's packed prefill, on ragged length mixes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def run_case(gpu, cfg, lengths, Hq, Hkv, D, W, dtype, max_seqlen=None):
    q, k, v, sink, cu = inputs.packed_inputs(cfg, 0, lengths, Hq, Hkv, D, dtype)
    ref_out, ref_lse = oracle.prefill_varlen(to64(q), to64(k), to64(v), to64(sink),
                                             cu.numpy(), W)
    S = max(lengths) if max_seqlen is None else max_seqlen
    print("varlen case", cfg, lengths, Hq, Hkv, D, W, dtype, flush=True)
    out, lse = swa.swa_sink_prefill_varlen(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu),
                                           cu.to(gpu), S, W)
    torch.cuda.synchronize()
    check_out(out, ref_out, dtype)
    check_lse(lse, ref_lse, dtype)
    return out, lse


CASES = [
    # lengths, Hq, Hkv, D, W
    ([300, 1, 0, 33, 64, 257], 8, 1, 128, 128),
    ([100, 31, 32, 200], 16, 2, 64, 128),
    ([129, 7, 96], 8, 2, 128, 33),
    ([500, 12], 64, 8, 128, 128),
    ([0, 0, 45], 4, 4, 128, 1),
    ([150, 90, 211], 8, 1, 128, 100000),      # window past every length: causal per sequence
    ([64, 64, 64, 64], 6, 2, 64, 64),
    ([77, 300, 1], 4, 2, 128, 128),            # packed ring kernel, GQA group 2
    ([65, 129, 0, 250], 8, 2, 64, 100),        # packed ring kernel, group 4, D=64, window 100
    ([40, 700], 4, 4, 128, 98),                # packed ring kernel, group 1, shortest ring window
]


@pytest.mark.parametrize("lengths,Hq,Hkv,D,W", CASES)
def test_bf16_against_oracle(gpu, lengths, Hq, Hkv, D, W):
    run_case(gpu, 95, lengths, Hq, Hkv, D, W, torch.bfloat16)


def test_f32_against_oracle(gpu):
    run_case(gpu, 96, [70, 3, 0, 130], 6, 2, 128, 40, torch.float32)


def test_max_seqlen_above_every_length(gpu):
    """Work-groups past each sequence's end exit without writing."""
    run_case(gpu, 97, [40, 90], 8, 1, 128, 128, torch.bfloat16, max_seqlen=400)


def test_many_short_sequences(gpu):
    """More than 64 sequences (several scan batches), most shorter than one
    work-group's share, so work-groups run many segments each."""
    lengths = [int(n) for n in inputs.cache_lengths(150, 0, 90, seed=9701)]
    run_case(gpu, 94, lengths, 8, 1, 128, 128, torch.bfloat16)
    run_case(gpu, 94, lengths, 8, 2, 64, 40, torch.bfloat16)


@pytest.mark.parametrize("W", [128, 57])
def test_uniform_pack_matches_batched_prefill(gpu, W):
    """Equal lengths: the pack is the [B, S] batch.  Every 32-row step of
    both entry points runs the same arithmetic on the same tiles (the split
    into work-groups differs), so the results are bit-identical."""
    B, S, Hq, Hkv, D = 3, 1190, 8, 2, 128
    q, k, v, sink = inputs.attention_inputs(98, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, gpu)
    cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32, device=gpu)
    o1, l1 = swa.swa_sink_prefill(q, k, v, sink, W)
    o2, l2 = swa.swa_sink_prefill_varlen(q.reshape(B * S, Hq, D), k.reshape(B * S, Hkv, D),
                                         v.reshape(B * S, Hkv, D), sink, cu, S, W)
    torch.cuda.synchronize()
    assert torch.equal(o1.reshape(B * S, Hq, D), o2)
    assert torch.equal(l1.permute(1, 0, 2).reshape(Hq, B * S), l2)


def test_rows_outside_sequences_untouched(gpu):
    """Rows past cu_seqlens[B] belong to no sequence and are never written."""
    lengths = [50, 20]
    q, k, v, sink, cu = inputs.packed_inputs(99, 0, lengths + [30], 8, 1, 128, torch.bfloat16,
                                             gpu)
    cu = cu[:3].contiguous()                    # the last 30 rows are not in the batch
    out = torch.full_like(q, 7.0)
    lse = torch.full((8, q.shape[0]), 7.0, device=gpu)
    swa.swa_sink_prefill_varlen(q, k, v, sink, cu, 50, 128, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out[70:] == 7.0) and torch.all(lse[:, 70:] == 7.0)
    assert torch.all(out[:70] != 7.0)


@pytest.mark.parametrize("global_layer", [False, True])
def test_bucket_full_size_sampled_rows(gpu, global_layer):
    """The benchmarked bucket (16 sequences, lengths uniform in [512, 8192],
    Hq=64, Hkv=8, D=128), as bench.py launches it: every sequence's first two
    and last two rows and six seeded random rows, all heads, against the
    oracle over that sequence's own keys."""
    Hq, Hkv, D = 64, 8, 128
    lengths = [int(n) for n in inputs.cache_lengths(16, 512, 8192, seed=6000)]
    S_max = max(lengths)
    W = S_max if global_layer else 128
    q, k, v, sink, cu = inputs.packed_inputs(6, 0, lengths, Hq, Hkv, D, torch.bfloat16, gpu)
    print("varlen bucket", "global" if global_layer else "window 128", flush=True)
    out, lse = swa.swa_sink_prefill_varlen(q, k, v, sink, cu, S_max, W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6001)
    offs = np.concatenate([[0], np.cumsum(lengths)])
    for b, n in enumerate(lengths):
        s0 = int(offs[b])
        pos = np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.integers(0, n, 6)]))
        idx = torch.as_tensor(s0 + pos, device=gpu)
        ref_out, ref_lse = oracle.swa_prefill_rows(
            to64(q.index_select(0, idx)), np.zeros(len(pos)), pos, to64(k[s0:s0 + n][None]),
            to64(v[s0:s0 + n][None]), to64(sink), W)
        check_out(out.index_select(0, idx), ref_out, torch.bfloat16)
        check_lse(lse.index_select(1, idx).T, ref_lse, torch.bfloat16)


@pytest.mark.parametrize("W", [128, 33])
def test_table_entries_are_clamped(gpu, W):
    """Offsets below 0 or past `total` are clamped by the kernels (no access
    leaves the tensors): [-5, 30, 500] over 100 rows runs as [0, 30, 100]."""
    lengths = [30, 70]
    q, k, v, sink, cu = inputs.packed_inputs(93, 0, lengths, 8, 2, 128, torch.bfloat16)
    ref_out, ref_lse = oracle.prefill_varlen(to64(q), to64(k), to64(v), to64(sink), cu.numpy(), W)
    bad = torch.tensor([-5, 30, 500], dtype=torch.int32)
    out, lse = swa.swa_sink_prefill_varlen(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu),
                                           bad.to(gpu), 70, W)
    torch.cuda.synchronize()
    check_out(out, ref_out, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)
