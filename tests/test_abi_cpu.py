"""The C ABI library loads, exports what include/swa_sink.h declares, and
rejects bad arguments before any HIP call (CPU only, no compute).

Every call here carries at least one invalid argument, so validation must
return before anything is launched; the pointers are dummies.
"""
from __future__ import annotations

import os
import re

import pytest

from sliding_window_learnable_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa_sink.h")

P = 4096          # a 16-byte-aligned dummy address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from sliding_window_learnable_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return set(re.findall(r"SWA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text))


def test_exports_every_declared_symbol(lib):
    declared = declared_functions()
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, val in [("SWA_OK", 0), ("SWA_ERR_NULL", -1), ("SWA_ERR_SHAPE", -2),
                      ("SWA_ERR_UNSUPPORTED", -3), ("SWA_ERR_WORKSPACE", -4),
                      ("SWA_ERR_HIP", -5), ("SWA_ERR_SCRATCH", -6), ("SWA_F32", 0),
                      ("SWA_BF16", 1)]:
        assert re.search(r"\b%s\s*=\s*%d\b" % (name, val), text), name
        assert getattr(_lib, name) == val


def test_strerror_every_code(lib):
    seen = set()
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = lib.swa_sink_strerror(code).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.swa_sink_strerror(12345).decode() == "unknown status code"


def prefill(lib, q=P, k=P, v=P, sink=P, out=P, lse=None, B=1, Hq=8, Hkv=1, S=16, D=128,
            window=128, dtype=1):
    return lib.swa_sink_prefill(q, k, v, sink, out, lse, B, Hq, Hkv, S, D, window, dtype, None)


def decode(lib, q=P, kc=P, vc=P, sink=P, out=P, lse=None, B=1, Hq=8, Hkv=1, T=1, W=128, D=128,
           cache_len=None, dtype=1):
    return lib.swa_sink_decode(q, kc, vc, sink, out, lse, B, Hq, Hkv, T, W, D, cache_len,
                               dtype, None)


def gattn(lib, q=P, k=P, v=P, sink=P, out=P, lse=None, B=1, Hq=8, Hkv=1, Sq=4, Skv=64, D=128,
          ws=None, wsb=0, dtype=1):
    return lib.global_sink_attn(q, k, v, sink, out, lse, B, Hq, Hkv, Sq, Skv, D, ws, wsb,
                                dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SWA_ERR_NULL), (dict(k=None), _lib.SWA_ERR_NULL),
    (dict(v=None), _lib.SWA_ERR_NULL), (dict(sink=None), _lib.SWA_ERR_NULL),
    (dict(out=None), _lib.SWA_ERR_NULL),
    (dict(B=-1), _lib.SWA_ERR_SHAPE), (dict(S=-3), _lib.SWA_ERR_SHAPE),
    (dict(Hq=0), _lib.SWA_ERR_SHAPE), (dict(Hkv=0), _lib.SWA_ERR_SHAPE),
    (dict(Hq=8, Hkv=3), _lib.SWA_ERR_SHAPE), (dict(window=0), _lib.SWA_ERR_SHAPE),
    (dict(D=0), _lib.SWA_ERR_SHAPE), (dict(B=70000), _lib.SWA_ERR_SHAPE),
    (dict(D=96), _lib.SWA_ERR_UNSUPPORTED), (dict(D=256), _lib.SWA_ERR_UNSUPPORTED),
    (dict(dtype=2), _lib.SWA_ERR_UNSUPPORTED), (dict(dtype=-1), _lib.SWA_ERR_UNSUPPORTED),
    (dict(q=P + 8), _lib.SWA_ERR_UNSUPPORTED), (dict(out=P + 2), _lib.SWA_ERR_UNSUPPORTED),
    (dict(lse=P + 2), _lib.SWA_ERR_UNSUPPORTED),
    # more 32-row work units than one launch grid holds
    (dict(B=60000, Hq=64, Hkv=8, S=1 << 30), _lib.SWA_ERR_SHAPE),
])
def test_prefill_rejects(lib, kw, code):
    assert prefill(lib, **kw) == code


def test_empty_inputs_are_noops(lib):
    # B == 0 or S == 0: nothing to compute, nothing launched, success
    assert prefill(lib, B=0) == _lib.SWA_OK
    assert prefill(lib, S=0) == _lib.SWA_OK
    assert decode(lib, B=0) == _lib.SWA_OK
    assert decode(lib, T=0) == _lib.SWA_OK
    assert gattn(lib, Sq=0) == _lib.SWA_OK
    assert gattn(lib, Sq=0, Skv=0) == _lib.SWA_OK


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SWA_ERR_NULL), (dict(kc=None), _lib.SWA_ERR_NULL),
    (dict(vc=None), _lib.SWA_ERR_NULL), (dict(sink=None), _lib.SWA_ERR_NULL),
    (dict(out=None), _lib.SWA_ERR_NULL),
    (dict(T=5, W=4), _lib.SWA_ERR_SHAPE), (dict(W=0), _lib.SWA_ERR_SHAPE),
    (dict(T=-1), _lib.SWA_ERR_SHAPE), (dict(Hq=6, Hkv=4), _lib.SWA_ERR_SHAPE),
    (dict(D=32), _lib.SWA_ERR_UNSUPPORTED), (dict(dtype=7), _lib.SWA_ERR_UNSUPPORTED),
    (dict(cache_len=P + 1), _lib.SWA_ERR_UNSUPPORTED), (dict(kc=P + 4), _lib.SWA_ERR_UNSUPPORTED),
    (dict(B=65535, Hq=65535, Hkv=1, T=1), _lib.SWA_ERR_SHAPE),       # B*Hq*T_q > 2^31-1
    (dict(W=(1 << 23) + 1, D=128), _lib.SWA_ERR_UNSUPPORTED),       # one ring above 2 GiB
])
def test_decode_rejects(lib, kw, code):
    assert decode(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SWA_ERR_NULL), (dict(sink=None), _lib.SWA_ERR_NULL),
    (dict(Sq=65, Skv=64), _lib.SWA_ERR_SHAPE), (dict(Skv=-1), _lib.SWA_ERR_SHAPE),
    (dict(Hq=5, Hkv=2), _lib.SWA_ERR_SHAPE),
    (dict(D=100), _lib.SWA_ERR_UNSUPPORTED), (dict(dtype=3), _lib.SWA_ERR_UNSUPPORTED),
    (dict(B=4, Hq=64, Hkv=8, Sq=1 << 30, Skv=1 << 30), _lib.SWA_ERR_SHAPE),
])
def test_global_rejects(lib, kw, code):
    assert gattn(lib, **kw) == code


def test_global_workspace_checked(lib):
    """Decode-shaped global calls split the keys and need a workspace."""
    need = lib.global_sink_attn_workspace_bytes(8, 64, 8, 1, 262144, 128)
    assert need > 0
    assert gattn(lib, B=8, Hq=64, Hkv=8, Sq=1, Skv=262144, ws=None, wsb=0) == _lib.SWA_ERR_WORKSPACE
    assert gattn(lib, B=8, Hq=64, Hkv=8, Sq=1, Skv=262144, ws=P, wsb=need - 1) == \
        _lib.SWA_ERR_WORKSPACE
    # a split's key range stays below 2 GiB of K rows: B=256 sequences fill the
    # GPU without splitting, but 2M-token caches (4 GiB of K per sequence) are
    # cut in two: 2 splits x 256 x 64 heads x 1 row x (128 + 2) floats
    assert lib.global_sink_attn_workspace_bytes(256, 64, 8, 1, 1 << 21, 128) == 2 * 256 * 64 * 130 * 4
    assert lib.global_sink_attn_workspace_bytes(256, 64, 8, 1, 1 << 20, 128) == 1 * 256 * 64 * 130 * 4
    # invalid sizes report no workspace
    assert lib.global_sink_attn_workspace_bytes(8, 64, 8, 5, 4, 128) == 0
    assert lib.global_sink_attn_workspace_bytes(8, 64, 8, 1, 4096, 96) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    import sliding_window_learnable_amd as swa
    q = torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        swa.swa_sink_prefill(q, k, k, torch.zeros(8), 128)


def test_binding_checks_caller_buffers():
    """Output buffers the caller passes must match the shapes the call writes
    (checked before anything reaches the library, so CPU tensors suffice)."""
    import torch
    import sliding_window_learnable_amd as swa
    bf = torch.bfloat16
    q = torch.zeros(2, 40, 8, 128, dtype=bf)
    k = torch.zeros(2, 40, 2, 128, dtype=bf)
    sink = torch.zeros(8)
    cases = [
        lambda: swa.swa_sink_prefill(q, k, k, sink, 128, out=torch.zeros(2, 39, 8, 128, dtype=bf)),
        lambda: swa.swa_sink_prefill(q, k, k, sink, 128, out=torch.zeros_like(q, dtype=torch.float32)),
        lambda: swa.swa_sink_prefill(q, k, k, sink, 128, lse=torch.zeros(2, 40, 8)),
        lambda: swa.global_sink_attn(q, k, k, sink, lse=torch.zeros(2, 8, 40, dtype=torch.float64)),
        lambda: swa.global_sink_attn_block_max(q, k, k, sink, 128, block_max=torch.zeros(2, 8, 2, 2)),
        lambda: swa.swa_sink_prefill_varlen(q[0], k[0], k[0], sink,
                                            torch.tensor([0, 40], dtype=torch.int32), 40, 128,
                                            lse=torch.zeros(40, 8)),
        lambda: swa.swa_sink_decode(q[:, :2], k.permute(0, 2, 1, 3).contiguous(),
                                    k.permute(0, 2, 1, 3).contiguous(), sink,
                                    lse=torch.zeros(2, 8, 3)),
        lambda: swa.swa_sink_rope_append(q[:, :2], k[:, :2], k[:, :2],
                                         k.permute(0, 2, 1, 3).contiguous(),
                                         k.permute(0, 2, 1, 3).contiguous(),
                                         q_rot=torch.zeros(2, 2, 8, 64, dtype=bf)),
        lambda: swa.swa_sink_backward(q, k, k, sink, q, torch.zeros(2, 8, 40), q, 128,
                                      dk=torch.zeros(2, 40, 8, 128, dtype=bf)),
        lambda: swa.swa_sink_backward(q, k, k, sink, q, torch.zeros(2, 8, 40), q, 128,
                                      dsink=torch.zeros(8, dtype=torch.float64)),
    ]
    for i, call in enumerate(cases):
        with pytest.raises(ValueError):
            call()
    with pytest.raises(TypeError):               # the sink is float32
        swa.global_sink_attn(q, k, k, sink.double())


def bwd(lib, q=P, k=P, v=P, sink=P, out=P, lse=P, dout=P, dq=P, dk=P, dv=P, dsink=P, B=1, Hq=8,
        Hkv=1, S=16, D=128, window=128, ws=P, wsb=1 << 20, dtype=1):
    return lib.swa_sink_backward(q, k, v, sink, out, lse, dout, dq, dk, dv, dsink, B, Hq, Hkv, S, D,
                                 window, ws, wsb, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SWA_ERR_NULL), (dict(lse=None), _lib.SWA_ERR_NULL),
    (dict(dout=None), _lib.SWA_ERR_NULL), (dict(dk=None), _lib.SWA_ERR_NULL),
    (dict(dsink=None), _lib.SWA_ERR_NULL), (dict(out=None), _lib.SWA_ERR_NULL),
    (dict(S=-1), _lib.SWA_ERR_SHAPE), (dict(window=0), _lib.SWA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), _lib.SWA_ERR_SHAPE), (dict(B=70000), _lib.SWA_ERR_SHAPE),
    (dict(D=48), _lib.SWA_ERR_UNSUPPORTED), (dict(dtype=9), _lib.SWA_ERR_UNSUPPORTED),
    (dict(dq=P + 8), _lib.SWA_ERR_UNSUPPORTED), (dict(dsink=P + 2), _lib.SWA_ERR_UNSUPPORTED),
    (dict(ws=None), _lib.SWA_ERR_WORKSPACE), (dict(wsb=16), _lib.SWA_ERR_WORKSPACE),
    (dict(ws=P + 4), _lib.SWA_ERR_UNSUPPORTED),
])
def test_backward_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_backward_workspace_and_empty(lib):
    # D_i and lse*log2(e) per (b, h, row) plus one sink-gradient partial per 32 rows, float32
    assert lib.swa_sink_backward_workspace_bytes(2, 64, 1000) == 4 * 2 * 64 * (2 * 1000 + 32)
    assert lib.swa_sink_backward_workspace_bytes(0, 64, 1000) == 0
    assert bwd(lib, B=0, ws=None, wsb=0) == _lib.SWA_OK
    assert bwd(lib, S=0, ws=None, wsb=0) == _lib.SWA_OK


def bmax(lib, q=P, k=P, v=P, sink=P, out=P, lse=None, bm=P, bk=128, B=1, Hq=8, Hkv=1, Sq=64,
         Skv=64, D=128, dtype=1):
    return lib.global_sink_attn_block_max(q, k, v, sink, out, lse, bm, bk, B, Hq, Hkv, Sq, Skv, D,
                                          dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SWA_ERR_NULL), (dict(bm=None), _lib.SWA_ERR_NULL),
    (dict(out=None), _lib.SWA_ERR_NULL),
    (dict(bk=0), _lib.SWA_ERR_SHAPE), (dict(bk=48), _lib.SWA_ERR_SHAPE),
    (dict(bk=16), _lib.SWA_ERR_SHAPE), (dict(Sq=65), _lib.SWA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), _lib.SWA_ERR_SHAPE),
    (dict(dtype=0), _lib.SWA_ERR_UNSUPPORTED), (dict(D=96), _lib.SWA_ERR_UNSUPPORTED),
    (dict(bm=P + 2), _lib.SWA_ERR_UNSUPPORTED), (dict(q=P + 8), _lib.SWA_ERR_UNSUPPORTED),
])
def test_block_max_rejects(lib, kw, code):
    assert bmax(lib, **kw) == code


def test_block_max_empty_is_noop(lib):
    assert bmax(lib, B=0) == _lib.SWA_OK
    assert bmax(lib, Sq=0) == _lib.SWA_OK


def dring(lib, q=P, kc=P, vc=P, sink=P, out=P, lse=None, B=1, Hq=8, Hkv=1, T=4, W=128, R=131,
          D=128, cache_len=None, dtype=1):
    return lib.swa_sink_decode_ring(q, kc, vc, sink, out, lse, B, Hq, Hkv, T, W, R, D, cache_len,
                                    dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SWA_ERR_NULL), (dict(out=None), _lib.SWA_ERR_NULL),
    (dict(W=0), _lib.SWA_ERR_SHAPE), (dict(R=100), _lib.SWA_ERR_SHAPE),
    (dict(T=132), _lib.SWA_ERR_SHAPE), (dict(T=-1), _lib.SWA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), _lib.SWA_ERR_SHAPE),
    (dict(D=80), _lib.SWA_ERR_UNSUPPORTED), (dict(dtype=4), _lib.SWA_ERR_UNSUPPORTED),
    (dict(cache_len=P + 2), _lib.SWA_ERR_UNSUPPORTED), (dict(kc=P + 8), _lib.SWA_ERR_UNSUPPORTED),
])
def test_decode_ring_rejects(lib, kw, code):
    assert dring(lib, **kw) == code


def rapp(lib, q=P, kn=P, vn=P, qr=P, kc=P, vc=P, cl=None, B=1, Hq=8, Hkv=1, T=4, R=131, D=128,
         theta=10000.0, dtype=1):
    return lib.swa_sink_rope_append(q, kn, vn, qr, kc, vc, cl, B, Hq, Hkv, T, R, D, theta, dtype,
                                    None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SWA_ERR_NULL), (dict(qr=None), _lib.SWA_ERR_NULL),
    (dict(kc=None), _lib.SWA_ERR_NULL),
    (dict(T=132), _lib.SWA_ERR_SHAPE), (dict(R=0), _lib.SWA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), _lib.SWA_ERR_SHAPE),
    (dict(theta=1.0), _lib.SWA_ERR_UNSUPPORTED), (dict(theta=float("nan")), _lib.SWA_ERR_UNSUPPORTED),
    (dict(D=96), _lib.SWA_ERR_UNSUPPORTED), (dict(dtype=2), _lib.SWA_ERR_UNSUPPORTED),
    (dict(vn=P + 8), _lib.SWA_ERR_UNSUPPORTED), (dict(cl=P + 1), _lib.SWA_ERR_UNSUPPORTED),
])
def test_rope_append_rejects(lib, kw, code):
    assert rapp(lib, **kw) == code


def test_ring_calls_empty_are_noops(lib):
    assert dring(lib, B=0) == _lib.SWA_OK and dring(lib, T=0) == _lib.SWA_OK
    assert rapp(lib, B=0) == _lib.SWA_OK and rapp(lib, T=0) == _lib.SWA_OK


def pvar(lib, q=P, k=P, v=P, sink=P, out=P, lse=None, cu=P, B=3, S=40, total=70, Hq=8, Hkv=1,
         D=128, window=128, dtype=1):
    return lib.swa_sink_prefill_varlen(q, k, v, sink, out, lse, cu, B, S, total, Hq, Hkv, D,
                                       window, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SWA_ERR_NULL), (dict(cu=None), _lib.SWA_ERR_NULL),
    (dict(out=None), _lib.SWA_ERR_NULL),
    (dict(B=-1), _lib.SWA_ERR_SHAPE), (dict(S=-1), _lib.SWA_ERR_SHAPE),
    (dict(total=-5), _lib.SWA_ERR_SHAPE), (dict(window=0), _lib.SWA_ERR_SHAPE),
    (dict(Hq=8, Hkv=3), _lib.SWA_ERR_SHAPE), (dict(B=70000), _lib.SWA_ERR_SHAPE),
    (dict(B=60000, Hq=64, Hkv=8, S=1 << 30), _lib.SWA_ERR_SHAPE),
    (dict(D=96), _lib.SWA_ERR_UNSUPPORTED), (dict(dtype=3), _lib.SWA_ERR_UNSUPPORTED),
    (dict(cu=P + 2), _lib.SWA_ERR_UNSUPPORTED), (dict(k=P + 8), _lib.SWA_ERR_UNSUPPORTED),
])
def test_prefill_varlen_rejects(lib, kw, code):
    assert pvar(lib, **kw) == code


def test_prefill_varlen_empty_is_noop(lib):
    assert pvar(lib, B=0) == _lib.SWA_OK
    assert pvar(lib, S=0) == _lib.SWA_OK
    assert pvar(lib, total=0) == _lib.SWA_OK


def test_noalloc_rejects_sizes_beyond_its_static_scratch(lib):
    """global_sink_attn_noalloc checks the split partials' size against its
    64 MiB static array before any HIP call: 4096 single-token rows of 64
    heads need 4096 * 64 * 130 * 4 bytes (136 MB).  Argument errors come
    first, as in global_sink_attn."""
    f = lib.global_sink_attn_noalloc
    need = lib.global_sink_attn_workspace_bytes(4096, 64, 8, 1, 65536, 128)
    assert need > 64 << 20
    assert f(P, P, P, P, P, P, 4096, 64, 8, 1, 65536, 128, _lib.SWA_BF16, None) == \
        _lib.SWA_ERR_SCRATCH
    assert f(None, P, P, P, P, P, 4096, 64, 8, 1, 65536, 128, 1, None) == _lib.SWA_ERR_NULL
    assert f(P, P, P, P, P, P, 4, 64, 8, 2, 1, 128, 1, None) == _lib.SWA_ERR_SHAPE
    assert f(P, P, P, P, P, P, 4, 64, 8, 1, 10, 96, 1, None) == _lib.SWA_ERR_UNSUPPORTED
    assert f(P, P, P, P, P, P, 0, 64, 8, 1, 10, 128, 1, None) == _lib.SWA_OK
    # just inside the limit: the size is accepted (nothing launched here:
    # validation only, the sizes are checked against the workspace formula)
    assert lib.global_sink_attn_workspace_bytes(8, 64, 8, 4, 262144, 128) <= 64 << 20
