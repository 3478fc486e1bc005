"""GPU parity: swa_sink_backward (HIP, through the C ABI) against the fp64
oracle's backward, on the same seeded inputs.  The forward's out and lse come
from the HIP forward, as they would in training.

bf16 bar per gradient: the larger of the N(0,1) bar (5e-2 of rms + |ref|)
and 1.25x the error of the fp64 model of the kernels' rounding points on the
same inputs (tests/bf16_model.py) -- on some shapes (D = 64 with a 300-key
window) those rounding points alone pass 5e-2, and a correct kernel lands on
the model's error to three digits."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_learnable_amd as swa
from sliding_window_learnable_amd import inputs
from tests.bf16_model import rounded_backward, scaled_error
from tests.parity import GRAD_C, check_grad, to64

pytestmark = pytest.mark.gpu


def forward_backward(q, k, v, sink, g, W):
    if W >= q.shape[1]:
        out, lse = swa.global_sink_attn(q, k, v, sink)
    else:
        out, lse = swa.swa_sink_prefill(q, k, v, sink, W)
    grads = swa.swa_sink_backward(q, k, v, sink, out, lse, g, W)
    torch.cuda.synchronize()
    return out, lse, grads


def bwd_case(gpu, cfg, B, S, Hq, Hkv, D, W, dtype, sink_override=None):
    q, k, v, sink = inputs.attention_inputs(cfg, 0, B, S, S, Hq, Hkv, D, dtype)
    g = inputs.upstream_grad(cfg, 0, B, S, Hq, D, dtype)
    if sink_override is not None:
        sink = torch.full((Hq,), float(sink_override))
    _, _, got = forward_backward(q.to(gpu), k.to(gpu), v.to(gpu), sink.to(gpu), g.to(gpu), W)
    args = (to64(q), to64(k), to64(v), to64(sink), to64(g), W)
    ref = oracle.attend_backward(*args)
    model = rounded_backward(*args) if dtype == torch.bfloat16 else None
    for n, (name, a, r) in enumerate(zip(("dq", "dk", "dv", "dsink"), got, ref)):
        c = None
        if model is not None and name != "dsink":
            c = max(GRAD_C[dtype], 1.25 * scaled_error(model[n], r))
        check_grad(a, r, dtype, name, c=c)
    return got, ref


CASES = [
    # B, S, Hq, Hkv, D, W
    (2, 150, 6, 2, 128, 33),
    (1, 97, 8, 8, 64, 200),        # window >= S: global causal
    (2, 300, 8, 1, 128, 128),
    (1, 1000, 64, 8, 128, 128),
    (3, 77, 4, 2, 64, 1),          # every row sees only itself
    (1, 333, 16, 2, 128, 100),
    (1, 200, 16, 1, 128, 128),     # two query heads per wave (G = 16)
    (2, 130, 32, 2, 64, 64),       # G = 16 at D = 64
    # key-tile ring (D = 128, window <= 129): one query head per KV head, so
    # a slot's next tile is needed in the step it retires; two heads; the
    # widest ring window; a two-tile window
    (1, 700, 4, 4, 128, 128),
    (1, 520, 4, 2, 128, 129),
    (2, 450, 8, 8, 128, 33),
    # windows above 256: four key tiles per dk/dv work-group (two below)
    (1, 600, 8, 2, 64, 300),
    (1, 400, 16, 1, 128, 400),     # global, G = 16
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,W", CASES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_backward_against_oracle(gpu, B, S, Hq, Hkv, D, W, dtype):
    bwd_case(gpu, 70, B, S, Hq, Hkv, D, W, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_backward_sink_neg_inf(gpu, dtype):
    got, _ = bwd_case(gpu, 71, 1, 200, 8, 2, 128, 128, dtype, sink_override=-np.inf)
    assert bool((got[3] == 0).all())


def test_backward_global_long(gpu):
    """Global causal backward over 2048 tokens (bf16)."""
    bwd_case(gpu, 72, 1, 2048, 16, 2, 128, 2048, torch.bfloat16)


def test_backward_deterministic(gpu):
    B, S, Hq, Hkv, D, W = 1, 700, 16, 2, 128, 128
    q, k, v, sink = inputs.attention_inputs(73, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    g = inputs.upstream_grad(73, 0, B, S, Hq, D, torch.bfloat16, "cuda")
    _, _, a = forward_backward(q, k, v, sink, g, W)
    _, _, b = forward_backward(q, k, v, sink, g, W)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_32k_slices_and_sink_identity(gpu):
    """The 32K prefill workload at full size (B=1, S=32768, Hq=64, Hkv=8,
    D=128, window 128).  Gradients of rows/keys inside two slices are
    compared with the oracle run on those slices (a slice preceded by W-1
    context tokens has every row's window complete; keys at least W-1 before
    its end receive all their queries).  The sink gradient is checked against
    -sum e^{s - lse} (dO . O) from the forward's own outputs."""
    B, S, Hq, Hkv, D, W = 1, 32768, 64, 8, 128, 128
    q, k, v, sink = inputs.attention_inputs(2, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    g = inputs.upstream_grad(2, 0, B, S, Hq, D, torch.bfloat16, "cuda")
    out, lse, (dq, dk, dv, ds) = forward_backward(q, k, v, sink, g, W)
    for s0, n in ((0, 512), (20000, 640)):
        a = max(0, s0 - (W - 1))
        sl = slice(a, s0 + n)
        rq, rk, rv, _ = oracle.attend_backward(to64(q[:, sl]), to64(k[:, sl]), to64(v[:, sl]),
                                               to64(sink), to64(g[:, sl]), W)
        rows = slice(s0 - a, s0 - a + n)                 # complete windows
        keys = slice(s0 - a, s0 - a + n - (W - 1))       # complete query sets
        check_grad(dq[:, s0:s0 + n], rq[:, rows], torch.bfloat16, "dq")
        check_grad(dk[:, s0:s0 + n - (W - 1)], rk[:, keys], torch.bfloat16, "dk")
        check_grad(dv[:, s0:s0 + n - (W - 1)], rv[:, keys], torch.bfloat16, "dv")
    dot = (g.double() * out.double()).sum(-1).permute(0, 2, 1)              # B Hq S
    expect = -(torch.exp(sink.double()[None, :, None] - lse.double()) * dot).sum(dim=(0, 2))
    check_grad(ds, to64(expect), torch.float32, "dsink", c=1e-4)


def test_backward_262144_slices(gpu):
    """Window-128 backward at S=262144 (B=1, Hq=64, Hkv=8, D=128), where the
    dk/dv work-groups walk runs of 256 key tiles (8192 positions) rather than
    the 32 of the 32K workload.  Two slices against the oracle run on them:
    one across the boundary between the third and fourth runs (position
    24576) and the last 640 rows of the sequence; a slice preceded by W-1
    context tokens has every row's window complete, and keys at least W-1
    before its end receive all their queries."""
    B, S, Hq, Hkv, D, W = 1, 262144, 64, 8, 128, 128
    print("backward 262144", flush=True)
    q, k, v, sink = inputs.attention_inputs(9, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    g = inputs.upstream_grad(9, 0, B, S, Hq, D, torch.bfloat16, "cuda")
    _, _, (dq, dk, dv, _) = forward_backward(q, k, v, sink, g, W)
    for s0, n in ((24576 - 300, 640), (S - 640, 640)):
        a = max(0, s0 - (W - 1))
        sl = slice(a, s0 + n)
        rq, rk, rv, _ = oracle.attend_backward(to64(q[:, sl]), to64(k[:, sl]), to64(v[:, sl]),
                                               to64(sink), to64(g[:, sl]), W)
        rows = slice(s0 - a, s0 - a + n)                 # complete windows
        check_grad(dq[:, s0:s0 + n], rq[:, rows], torch.bfloat16, "dq")
        if s0 + n < S:
            keys = slice(s0 - a, s0 - a + n - (W - 1))   # complete query sets
            check_grad(dk[:, s0:s0 + n - (W - 1)], rk[:, keys], torch.bfloat16, "dk")
            check_grad(dv[:, s0:s0 + n - (W - 1)], rv[:, keys], torch.bfloat16, "dv")
        else:
            # the sequence's last keys: every query that sees them is inside the slice
            keys = slice(s0 - a, s0 - a + n)
            check_grad(dk[:, s0:], rk[:, keys], torch.bfloat16, "dk")
            check_grad(dv[:, s0:], rv[:, keys], torch.bfloat16, "dv")
