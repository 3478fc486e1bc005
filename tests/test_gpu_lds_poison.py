"""LDS-poisoning debug build against the product build, through the C ABI.

libswa_sink_poison.so is the same library built with SWA_LDS_POISON: its
kernels fill their LDS with NaN patterns on entry and overwrite every
buffer->LDS copy's destination with NaN just before the copy.  A kernel that
reads LDS nothing has written yet (a tile never staged, a slot read before
its copy landed because a wait or a barrier is missing, a stale slot index)
then produces NaN instead of plausible old values.  A correct kernel gives
bit-identical results in both builds, which is what every case checks, on
the paths that stage through LDS: the ring prefill (uniform and packed), the
streaming kernel (global, wide window, packed, block maxima), ring decode,
split-KV decode, the allocation-free global call and the backward."""
from __future__ import annotations

import os

import pytest
import torch

from sliding_window_learnable_amd import _lib, inputs

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
POISON = os.path.join(os.path.dirname(_lib.LIB_PATH), "libswa_sink_poison.so")


@pytest.fixture(scope="module")
def libs(gpu):
    if not os.path.exists(POISON):
        pytest.fail("libswa_sink_poison.so is not built (sliding_window_learnable_amd.build)")
    return _lib.load(), _lib.load(POISON)


def ptr(t):
    return None if t is None else t.data_ptr()


def stream():
    return torch.cuda.current_stream().cuda_stream


def same(outs_a, outs_b, what):
    torch.cuda.synchronize()
    for a, b in zip(outs_a, outs_b):
        assert not torch.isnan(a.float()).any(), "%s: NaN in the product build" % what
        assert torch.equal(a, b), "%s: debug build differs (%d elements, NaN: %d)" % (
            what, int((a != b).sum()), int(torch.isnan(b.float()).sum()))


def run_both(libs, fn):
    return [fn(lib) for lib in libs]


@pytest.mark.parametrize("B,S,Hq,Hkv,W", [(2, 1000, 64, 8, 128), (1, 32768, 64, 8, 128),
                                          (1, 700, 16, 2, 98), (1, 900, 16, 2, 511),
                                          (1, 777, 8, 1, 4096)])
def test_prefill(libs, B, S, Hq, Hkv, W):
    q, k, v, sink = inputs.attention_inputs(150, 0, B, S, S, Hq, Hkv, 128, BF16, "cuda")

    def call(lib):
        out, lse = torch.empty_like(q), torch.empty(B, Hq, S, device="cuda")
        assert lib.swa_sink_prefill(ptr(q), ptr(k), ptr(v), ptr(sink), ptr(out), ptr(lse), B, Hq,
                                    Hkv, S, 128, W, 1, stream()) == 0
        return out, lse

    a, b = run_both(libs, call)
    same(a, b, "prefill W=%d" % W)


@pytest.mark.parametrize("W", [128, 100000])
def test_prefill_varlen(libs, W):
    lengths = [300, 1, 0, 77, 2050, 33, 640]
    q, k, v, sink, cu = inputs.packed_inputs(151, 0, lengths, 64, 8, 128, BF16, "cuda")
    total = q.shape[0]

    def call(lib):
        out, lse = torch.empty_like(q), torch.empty(64, total, device="cuda")
        assert lib.swa_sink_prefill_varlen(ptr(q), ptr(k), ptr(v), ptr(sink), ptr(out), ptr(lse),
                                           ptr(cu), len(lengths), max(lengths), total, 64, 8, 128,
                                           W, 1, stream()) == 0
        return out, lse

    a, b = run_both(libs, call)
    same(a, b, "varlen W=%d" % W)


@pytest.mark.parametrize("Sq,Skv", [(2000, 2000), (1, 70000), (4, 9000), (65, 700)])
def test_global(libs, Sq, Skv):
    B, Hq, Hkv = 2, 64, 8
    q, k, v, sink = inputs.attention_inputs(152, 0, B, Sq, Skv, Hq, Hkv, 128, BF16, "cuda")
    need = libs[0].global_sink_attn_workspace_bytes(B, Hq, Hkv, Sq, Skv, 128)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def call(lib):
        out, lse = torch.empty_like(q), torch.empty(B, Hq, Sq, device="cuda")
        assert lib.global_sink_attn(ptr(q), ptr(k), ptr(v), ptr(sink), ptr(out), ptr(lse), B, Hq,
                                    Hkv, Sq, Skv, 128, ptr(ws), ws.numel(), 1, stream()) == 0
        out2, lse2 = torch.empty_like(q), torch.empty(B, Hq, Sq, device="cuda")
        assert lib.global_sink_attn_noalloc(ptr(q), ptr(k), ptr(v), ptr(sink), ptr(out2),
                                            ptr(lse2), B, Hq, Hkv, Sq, Skv, 128, 1,
                                            stream()) == 0
        return out, lse, out2, lse2

    a, b = run_both(libs, call)
    same(a, b, "global %dx%d" % (Sq, Skv))


def test_block_max(libs):
    B, S, Hq, Hkv = 1, 3000, 16, 2
    q, k, v, sink = inputs.attention_inputs(153, 0, B, S, S, Hq, Hkv, 128, BF16, "cuda")

    def call(lib):
        out, lse = torch.empty_like(q), torch.empty(B, Hq, S, device="cuda")
        bm = torch.empty(B, Hq, (S + 31) // 32, (S + 127) // 128, device="cuda")
        assert lib.global_sink_attn_block_max(ptr(q), ptr(k), ptr(v), ptr(sink), ptr(out),
                                              ptr(lse), ptr(bm), 128, B, Hq, Hkv, S, S, 128, 1,
                                              stream()) == 0
        return out, lse, bm

    a, b = run_both(libs, call)
    same(a, b, "block max")


@pytest.mark.parametrize("T,R", [(1, 128), (4, 128), (4, 131)])
def test_ring_decode(libs, T, R):
    B, Hq, Hkv = 64, 64, 8
    q, kc, vc, sink = inputs.ring_inputs(154, T, B, T, Hq, Hkv, R, 128, BF16, "cuda")
    lens = inputs.cache_lengths(B, 1, 3 * R, 154).to("cuda")

    def call(lib):
        out, lse = torch.empty_like(q), torch.empty(B, Hq, T, device="cuda")
        assert lib.swa_sink_decode_ring(ptr(q), ptr(kc), ptr(vc), ptr(sink), ptr(out), ptr(lse), B,
                                        Hq, Hkv, T, 128, R, 128, ptr(lens), 1, stream()) == 0
        return out, lse

    a, b = run_both(libs, call)
    same(a, b, "ring decode T=%d R=%d" % (T, R))


@pytest.mark.parametrize("S,W", [(1000, 128), (512, 512)])
def test_backward(libs, S, W):
    B, Hq, Hkv = 1, 16, 2
    q, k, v, sink = inputs.attention_inputs(155, 0, B, S, S, Hq, Hkv, 128, BF16, "cuda")
    g = inputs.upstream_grad(155, 0, B, S, Hq, 128, BF16, "cuda")
    out, lse = torch.empty_like(q), torch.empty(B, Hq, S, device="cuda")
    assert libs[0].swa_sink_prefill(ptr(q), ptr(k), ptr(v), ptr(sink), ptr(out), ptr(lse), B, Hq,
                                    Hkv, S, 128, W, 1, stream()) == 0
    need = libs[0].swa_sink_backward_workspace_bytes(B, Hq, S)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call(lib):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ds = torch.empty(Hq, device="cuda")
        assert lib.swa_sink_backward(ptr(q), ptr(k), ptr(v), ptr(sink), ptr(out), ptr(lse), ptr(g),
                                     ptr(dq), ptr(dk), ptr(dv), ptr(ds), B, Hq, Hkv, S, 128, W,
                                     ptr(ws), need, 1, stream()) == 0
        return dq, dk, dv, ds

    a, b = run_both(libs, call)
    same(a, b, "backward S=%d W=%d" % (S, W))
