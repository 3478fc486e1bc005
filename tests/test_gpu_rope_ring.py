"""GPU parity: swa_sink_rope_append and swa_sink_decode_ring against the
fp64 oracle through the C ABI, including a multi-step MTP draft loop with
random acceptance and rollback in a ring of window + T_q - 1 slots."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def gen(seed, shape, dtype, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("B,T,Hq,Hkv,R,D,lens", [
    (3, 4, 8, 1, 131, 128, [0, 200, 1_000_003]),
    (2, 1, 16, 2, 128, 64, [5, 127]),
    (2, 3, 6, 2, 100, 128, [262_141, 99]),
    # malformed (negative) cache lengths: slots are P mod ring in [0, ring),
    # so every write stays inside its own sequence's ring
    (3, 4, 8, 1, 131, 128, [-1, -5, -136]),
])
def test_rope_append_matches_oracle(gpu, dtype, B, T, Hq, Hkv, R, D, lens):
    q = gen(1, (B, T, Hq, D), dtype)
    kn = gen(2, (B, T, Hkv, D), dtype)
    vn = gen(3, (B, T, Hkv, D), dtype)
    kc0 = gen(4, (B, Hkv, R, D), dtype)
    vc0 = gen(5, (B, Hkv, R, D), dtype)
    cl = torch.tensor(lens, dtype=torch.int32)
    theta = 1e6 if D == 128 else 10000.0
    kc, vc = kc0.to(gpu), vc0.to(gpu)
    qr = swa.swa_sink_rope_append(q.to(gpu), kn.to(gpu), vn.to(gpu), kc, vc, cl.to(gpu), theta)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.rope_append(to64(q), to64(kn), to64(vn), to64(kc0), to64(vc0),
                                    cl.numpy(), theta)
    check_out(qr, rq, dtype, "q_rot")
    check_out(kc, rk, dtype, "kcache")
    # values are copied exactly; untouched slots keep their bits
    assert np.array_equal(to64(vc), rv)
    written = np.zeros((B, R), bool)
    for b in range(B):
        for t in range(T):
            written[b, (lens[b] + t) % R] = True
    keep = torch.as_tensor(~written)[:, None, :, None].expand(B, Hkv, R, D)
    assert torch.equal(kc.cpu()[keep], kc0[keep])


def test_rope_append_in_place(gpu):
    B, T, Hq, Hkv, R, D = 2, 4, 8, 1, 131, 128
    q = gen(6, (B, T, Hq, D), torch.bfloat16).to(gpu)
    kn = gen(7, (B, T, Hkv, D), torch.bfloat16).to(gpu)
    kc = torch.zeros((B, Hkv, R, D), dtype=torch.bfloat16, device=gpu)
    vc = torch.zeros_like(kc)
    ref = swa.swa_sink_rope_append(q, kn, kn, kc.clone(), vc.clone(), None, 10000.0)
    out = swa.swa_sink_rope_append(q, kn, kn, kc, vc, None, 10000.0, q_rot=q)
    torch.cuda.synchronize()
    assert out.data_ptr() == q.data_ptr() and torch.equal(q, ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("B,T,Hq,Hkv,W,R,D,lens", [
    (3, 4, 8, 1, 128, 131, 128, [131, 5000, 7]),
    (2, 4, 64, 8, 128, 131, 128, [1_000_003, 132]),
    (2, 2, 16, 2, 60, 100, 64, [100, 333]),
    (2, 1, 8, 1, 128, 128, 128, [128, 129]),
])
def test_decode_ring_matches_oracle(gpu, dtype, B, T, Hq, Hkv, W, R, D, lens):
    q, kc, vc, sink = inputs.ring_inputs(92, 0, B, T, Hq, Hkv, R, D, dtype)
    cl = torch.tensor(lens, dtype=torch.int32)
    out, lse = swa.swa_sink_decode_ring(q.to(gpu), kc.to(gpu), vc.to(gpu), sink.to(gpu), W,
                                        cl.to(gpu))
    torch.cuda.synchronize()
    ref, ref_lse = oracle.ring_decode(to64(q), to64(kc), to64(vc), to64(sink), cl.numpy(), window=W)
    check_out(out, ref, dtype)
    check_lse(lse, ref_lse.transpose(0, 2, 1), dtype)


def test_decode_ring_equal_sizes_is_swa_sink_decode(gpu):
    B, T, Hq, Hkv, W, D = 4, 4, 64, 8, 128, 128
    q, kc, vc, sink = inputs.ring_inputs(91, 0, B, T, Hq, Hkv, W, D, torch.bfloat16, gpu)
    cl = torch.tensor([128, 4, 1000, 131], dtype=torch.int32, device=gpu)
    a = swa.swa_sink_decode(q, kc, vc, sink, cl)
    b = swa.swa_sink_decode_ring(q, kc, vc, sink, W, cl)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_mtp_draft_loop_with_rollback(gpu):
    """40 steps of 1 + 3 drafts per sequence, a random number accepted per
    step and the rest rolled back, in rings of 131 slots with window 128:
    after each append the GPU ring equals the oracle's, and each step's
    decode (every draft seeing its full 128-key window) matches the oracle."""
    B, T, Hq, Hkv, W, D, steps, theta = 3, 4, 8, 1, 128, 128, 40, 1e6
    R = W + T - 1
    rng = np.random.default_rng(5)
    sink = gen(8, (Hq,), torch.float32)
    kc = torch.zeros((B, Hkv, R, D), dtype=torch.bfloat16, device=gpu)
    vc = torch.zeros_like(kc)
    okc, ovc = np.zeros((B, Hkv, R, D)), np.zeros((B, Hkv, R, D))
    L = np.zeros(B, dtype=np.int32)
    for s in range(steps):
        q = gen(100 + s, (B, T, Hq, D), torch.bfloat16)
        kn = gen(200 + s, (B, T, Hkv, D), torch.bfloat16)
        vn = gen(300 + s, (B, T, Hkv, D), torch.bfloat16)
        cl_old = torch.tensor(L, dtype=torch.int32)
        qr = swa.swa_sink_rope_append(q.to(gpu), kn.to(gpu), vn.to(gpu), kc, vc, cl_old.to(gpu),
                                      theta)
        out, lse = swa.swa_sink_decode_ring(qr, kc, vc, sink.to(gpu), W, (cl_old + T).to(gpu))
        torch.cuda.synchronize()
        rq, okc, ovc = oracle.rope_append(to64(q), to64(kn), to64(vn), okc, ovc, L, theta)
        check_out(kc, okc, torch.bfloat16, "kcache step %d" % s)
        assert np.array_equal(to64(vc), ovc)
        # decode parity on the GPU's own (bf16) inputs
        ref, ref_lse = oracle.ring_decode(to64(qr), to64(kc), to64(vc), to64(sink), L + T, window=W)
        check_out(out, ref, torch.bfloat16, "out step %d" % s)
        check_lse(lse, ref_lse.transpose(0, 2, 1), torch.bfloat16, "lse step %d" % s)
        okc, ovc = to64(kc), to64(vc)                 # follow the GPU's rounded cache
        L = L + rng.integers(1, T + 1, size=B).astype(np.int32)


def test_decode_ring_full_size(gpu):
    """Batched decode workload with a rollback ring: B=256, T_q=4, Hq=64,
    Hkv=8, D=128, window 128 in 131-slot rings, positions past the wrap."""
    B, T, Hq, Hkv, W, R, D = 256, 4, 64, 8, 128, 131, 128
    q, kc, vc, sink = inputs.ring_inputs(3, 1, B, T, Hq, Hkv, R, D, torch.bfloat16, gpu)
    cl = torch.tensor(np.random.default_rng(6).integers(R, 1 << 20, size=B), dtype=torch.int32,
                      device=gpu)
    out, lse = swa.swa_sink_decode_ring(q, kc, vc, sink, W, cl)
    torch.cuda.synchronize()
    for b in (0, 77, 255):
        ref, ref_lse = oracle.ring_decode(to64(q[b:b + 1]), to64(kc[b:b + 1]), to64(vc[b:b + 1]),
                                          to64(sink), cl[b:b + 1].cpu().numpy(), window=W)
        check_out(out[b:b + 1], ref, torch.bfloat16)
        check_lse(lse[b:b + 1], ref_lse.transpose(0, 2, 1), torch.bfloat16)
