"""MI355X-native sliding-window attention with a learnable per-head sink.

Thin Python binding over the C ABI of ``libswa_sink.so`` (hand-written HIP
kernels for gfx950).  The functions below only marshal arguments: they check
devices, dtypes and contiguity, allocate outputs with torch (device memory
plumbing), pass raw pointers plus the current HIP stream, and raise on a
non-zero status.  Every step of the computation runs in the HIP kernels.

Names follow the C entry points: ``swa_sink_prefill``, ``swa_sink_decode``,
``global_sink_attn`` (plus ``global_sink_attn_workspace_bytes``) and the
backward ``swa_sink_backward`` (plus ``swa_sink_backward_workspace_bytes``).
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import SwaError

__all__ = [
    "swa_sink_prefill",
    "swa_sink_prefill_varlen",
    "swa_sink_decode",
    "swa_sink_decode_ring",
    "swa_sink_rope_append",
    "global_sink_attn",
    "global_sink_attn_workspace_bytes",
    "global_sink_attn_noalloc",
    "global_sink_attn_block_max",
    "swa_sink_backward",
    "swa_sink_backward_workspace_bytes",
    "SwaError",
]

_DTYPES = {torch.float32: _lib.SWA_F32, torch.bfloat16: _lib.SWA_BF16}


def _dtype_code(*tensors) -> int:
    dt = tensors[0].dtype
    if dt not in _DTYPES:
        raise TypeError("q/k/v must be float32 or bfloat16, got %s" % dt)
    for t in tensors:
        if t.dtype != dt:
            raise TypeError("q, k, v and out must share one dtype")
    return _DTYPES[dt]


def _check_device(*tensors):
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("every tensor must be contiguous")


def _expect(t, shape, dtype, name):
    """A caller-provided buffer must have exactly the shape and dtype the call
    writes: the kernels trust the sizes they are given."""
    if t is not None and (tuple(t.shape) != tuple(shape) or t.dtype != dtype):
        raise ValueError("%s must be %s %s, got %s %s"
                         % (name, dtype, tuple(shape), t.dtype, tuple(t.shape)))


def _float32_sink(sink):
    if sink.dtype != torch.float32:
        raise TypeError("sink must be float32")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _call(fn, name, *args):
    rc = fn(*args)
    if rc != _lib.SWA_OK:
        raise SwaError(rc, name)


def swa_sink_prefill(q, k, v, sink, window: int, out=None, lse=None, want_lse: bool = True,
                     stream=None):
    """Causal sliding-window prefill.

    q [B, S, Hq, D], k/v [B, S, Hkv, D] (float32 or bfloat16), sink [Hq] float32.
    Returns (out [B, S, Hq, D], lse [B, Hq, S] float32 or None).
    """
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape or sink.shape != (Hq,):
        raise ValueError("shape mismatch: q %s k %s v %s sink %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape), tuple(sink.shape)))
    if sink.dtype != torch.float32:
        raise TypeError("sink must be float32")
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, S), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, S), device=q.device, dtype=torch.float32)
    _check_device(q, k, v, sink, out, lse)
    dt = _dtype_code(q, k, v, out)
    _call(_lib.load().swa_sink_prefill, "swa_sink_prefill", _ptr(q), _ptr(k), _ptr(v),
          _ptr(sink), _ptr(out), _ptr(lse), B, Hq, Hkv, S, D, int(window), dt, _stream(stream))
    return out, lse


def swa_sink_prefill_varlen(q, k, v, sink, cu_seqlens, max_seqlen: int, window: int, out=None,
                            lse=None, want_lse: bool = True, stream=None):
    """Sliding-window (or, with window >= max_seqlen, global causal) prefill
    over a packed batch: q [total, Hq, D], k/v [total, Hkv, D], cu_seqlens
    int32 [B + 1] on the GPU (sequence b is rows cu_seqlens[b] ..
    cu_seqlens[b+1] - 1, each at most max_seqlen long).
    Returns (out [total, Hq, D], lse [Hq, total] float32 or None).
    """
    total, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (total, Hkv, D) or v.shape != k.shape or sink.shape != (Hq,):
        raise ValueError("shape mismatch: q %s k %s v %s sink %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape), tuple(sink.shape)))
    if sink.dtype != torch.float32:
        raise TypeError("sink must be float32")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be int32 [B + 1]")
    B = cu_seqlens.numel() - 1
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (Hq, total), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((Hq, total), device=q.device, dtype=torch.float32)
    _check_device(q, k, v, sink, out, lse, cu_seqlens)
    dt = _dtype_code(q, k, v, out)
    _call(_lib.load().swa_sink_prefill_varlen, "swa_sink_prefill_varlen", _ptr(q), _ptr(k),
          _ptr(v), _ptr(sink), _ptr(out), _ptr(lse), _ptr(cu_seqlens), B, int(max_seqlen),
          total, Hq, Hkv, D, int(window), dt, _stream(stream))
    return out, lse


def swa_sink_decode(q, kcache, vcache, sink, cache_len=None, out=None, lse=None,
                    want_lse: bool = True, stream=None):
    """Decode T_q tokens per sequence over a W-slot ring cache.

    q [B, T_q, Hq, D]; kcache/vcache [B, Hkv, W, D] (key of position P in slot
    P % W); cache_len int32 [B] on the GPU (tokens written so far, including
    the T_q new ones) or None for full rings.  Returns (out, lse [B, Hq, T_q]).
    """
    B, T, Hq, D = q.shape
    Bk, Hkv, W, Dk = kcache.shape
    if Bk != B or Dk != D or vcache.shape != kcache.shape or sink.shape != (Hq,):
        raise ValueError("shape mismatch")
    if cache_len is not None and (cache_len.dtype != torch.int32 or cache_len.shape != (B,)):
        raise ValueError("cache_len must be int32 [B]")
    _float32_sink(sink)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, T), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), device=q.device, dtype=torch.float32)
    _check_device(q, kcache, vcache, sink, out, lse, cache_len)
    dt = _dtype_code(q, kcache, vcache, out)
    _call(_lib.load().swa_sink_decode, "swa_sink_decode", _ptr(q), _ptr(kcache), _ptr(vcache),
          _ptr(sink), _ptr(out), _ptr(lse), B, Hq, Hkv, T, W, D, _ptr(cache_len), dt,
          _stream(stream))
    return out, lse


def swa_sink_decode_ring(q, kcache, vcache, sink, window: int, cache_len=None, out=None, lse=None,
                         want_lse: bool = True, stream=None):
    """Ring decode with an attention window of ``window`` keys in a ring of
    R = kcache.shape[2] >= window slots (R >= window + T_q - 1 gives every
    draft its full window under rollback).  Query t at position
    p = L - T_q + t sees max(0, L - R, p - window + 1) .. p.
    Returns (out, lse [B, Hq, T_q])."""
    B, T, Hq, D = q.shape
    Bk, Hkv, R, Dk = kcache.shape
    if Bk != B or Dk != D or vcache.shape != kcache.shape or sink.shape != (Hq,):
        raise ValueError("shape mismatch")
    if cache_len is not None and (cache_len.dtype != torch.int32 or cache_len.shape != (B,)):
        raise ValueError("cache_len must be int32 [B]")
    _float32_sink(sink)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, T), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), device=q.device, dtype=torch.float32)
    _check_device(q, kcache, vcache, sink, out, lse, cache_len)
    dt = _dtype_code(q, kcache, vcache, out)
    _call(_lib.load().swa_sink_decode_ring, "swa_sink_decode_ring", _ptr(q), _ptr(kcache),
          _ptr(vcache), _ptr(sink), _ptr(out), _ptr(lse), B, Hq, Hkv, T, int(window), R, D,
          _ptr(cache_len), dt, _stream(stream))
    return out, lse


def swa_sink_rope_append(q, k_new, v_new, kcache, vcache, cache_len_old=None, rope_theta=10000.0,
                         q_rot=None, stream=None):
    """RoPE on the T_q new queries and keys at positions cache_len_old + t and
    the rotated keys and the values written to ring slots (position mod R) of
    kcache / vcache [B, Hkv, R, D] in place.  Returns q_rot [B, T_q, Hq, D]
    (``q_rot=q`` rotates in place)."""
    B, T, Hq, D = q.shape
    Bk, Hkv, R, Dk = kcache.shape
    if (k_new.shape != (B, T, Hkv, D) or v_new.shape != k_new.shape or Bk != B or Dk != D
            or vcache.shape != kcache.shape):
        raise ValueError("shape mismatch")
    if cache_len_old is not None and (cache_len_old.dtype != torch.int32
                                      or cache_len_old.shape != (B,)):
        raise ValueError("cache_len_old must be int32 [B]")
    _expect(q_rot, q.shape, q.dtype, "q_rot")
    if q_rot is None:
        q_rot = torch.empty_like(q)
    _check_device(q, k_new, v_new, kcache, vcache, q_rot, cache_len_old)
    dt = _dtype_code(q, k_new, v_new, kcache, vcache, q_rot)
    _call(_lib.load().swa_sink_rope_append, "swa_sink_rope_append", _ptr(q), _ptr(k_new),
          _ptr(v_new), _ptr(q_rot), _ptr(kcache), _ptr(vcache), _ptr(cache_len_old), B, Hq, Hkv,
          T, R, D, float(rope_theta), dt, _stream(stream))
    return q_rot


def global_sink_attn_workspace_bytes(B, Hq, Hkv, S_q, S_kv, D) -> int:
    return int(_lib.load().global_sink_attn_workspace_bytes(B, Hq, Hkv, S_q, S_kv, D))


def global_sink_attn(q, k, v, sink, out=None, lse=None, workspace=None, want_lse: bool = True,
                     stream=None):
    """Global causal attention, queries aligned to the end of the keys.

    q [B, S_q, Hq, D], k/v [B, S_kv, Hkv, D]; returns (out, lse [B, Hq, S_q]).
    ``workspace`` (a uint8 GPU tensor) is allocated when needed and not given.
    """
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Skv, Hkv, D) or v.shape != k.shape or sink.shape != (Hq,):
        raise ValueError("shape mismatch")
    _float32_sink(sink)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, Sq), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), device=q.device, dtype=torch.float32)
    need = global_sink_attn_workspace_bytes(B, Hq, Hkv, Sq, Skv, D)
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    _check_device(q, k, v, sink, out, lse, workspace)
    dt = _dtype_code(q, k, v, out)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call(_lib.load().global_sink_attn, "global_sink_attn", _ptr(q), _ptr(k), _ptr(v),
          _ptr(sink), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Skv, D, _ptr(workspace), wbytes,
          dt, _stream(stream))
    return out, lse


def global_sink_attn_noalloc(q, k, v, sink, out=None, lse=None, want_lse: bool = True,
                             stream=None):
    """global_sink_attn without a workspace: the library's static per-GPU
    scratch array holds the split partials (64 MiB; larger sizes raise).
    Calls overlapping on one GPU race on that array.  Outputs are allocated
    here when not given; the C call itself allocates nothing."""
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Skv, Hkv, D) or v.shape != k.shape or sink.shape != (Hq,):
        raise ValueError("shape mismatch")
    _float32_sink(sink)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, Sq), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), device=q.device, dtype=torch.float32)
    _check_device(q, k, v, sink, out, lse)
    dt = _dtype_code(q, k, v, out)
    _call(_lib.load().global_sink_attn_noalloc, "global_sink_attn_noalloc", _ptr(q), _ptr(k),
          _ptr(v), _ptr(sink), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Skv, D, dt,
          _stream(stream))
    return out, lse


def global_sink_attn_block_max(q, k, v, sink, block_k=128, out=None, lse=None, block_max=None,
                               want_lse: bool = True, stream=None):
    """global_sink_attn (bf16) plus, for every query head, 32-row query block
    and ``block_k``-key block, the largest scaled logit q.k/sqrt(D) over the
    block's visible pairs (-inf when none).

    Returns (out, lse, block_max [B, Hq, ceil(S_q/32), ceil(S_kv/block_k)]).
    """
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Skv, Hkv, D) or v.shape != k.shape or sink.shape != (Hq,):
        raise ValueError("shape mismatch")
    _float32_sink(sink)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, Sq), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), device=q.device, dtype=torch.float32)
    nkb = -(-Skv // block_k) if block_k > 0 else 0
    _expect(block_max, (B, Hq, -(-Sq // 32), nkb), torch.float32, "block_max")
    if block_max is None:
        block_max = torch.empty((B, Hq, -(-Sq // 32), nkb), device=q.device,
                                dtype=torch.float32)
    _check_device(q, k, v, sink, out, lse, block_max)
    dt = _dtype_code(q, k, v, out)
    _call(_lib.load().global_sink_attn_block_max, "global_sink_attn_block_max", _ptr(q), _ptr(k),
          _ptr(v), _ptr(sink), _ptr(out), _ptr(lse), _ptr(block_max), block_k, B, Hq, Hkv, Sq,
          Skv, D, dt, _stream(stream))
    return out, lse, block_max


def swa_sink_backward_workspace_bytes(B, Hq, S) -> int:
    return int(_lib.load().swa_sink_backward_workspace_bytes(B, Hq, S))


def swa_sink_backward(q, k, v, sink, out, lse, dout, window, dq=None, dk=None, dv=None,
                      dsink=None, workspace=None, stream=None):
    """Gradients of swa_sink_prefill (window < S) or of causal global attention
    (window >= S) for the upstream gradient ``dout``.

    q, out, dout [B, S, Hq, D]; k, v [B, S, Hkv, D]; sink [Hq]; lse [B, Hq, S]
    (the forward's outputs).  Returns (dq, dk, dv, dsink) with dsink [Hq]
    float32 summed over the batch.
    """
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if (k.shape != (B, S, Hkv, D) or v.shape != k.shape or sink.shape != (Hq,)
            or out.shape != q.shape or dout.shape != q.shape or lse.shape != (B, Hq, S)):
        raise ValueError("shape mismatch")
    _float32_sink(sink)
    _expect(lse, (B, Hq, S), torch.float32, "lse")
    _expect(dq, q.shape, q.dtype, "dq")
    _expect(dk, k.shape, k.dtype, "dk")
    _expect(dv, v.shape, v.dtype, "dv")
    _expect(dsink, (Hq,), torch.float32, "dsink")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dsink is None:
        dsink = torch.empty((Hq,), device=q.device, dtype=torch.float32)
    need = swa_sink_backward_workspace_bytes(B, Hq, S)
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    _check_device(q, k, v, sink, out, lse, dout, dq, dk, dv, dsink, workspace)
    dt = _dtype_code(q, k, v, out, dout, dq, dk, dv)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call(_lib.load().swa_sink_backward, "swa_sink_backward", _ptr(q), _ptr(k), _ptr(v),
          _ptr(sink), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(dsink), B, Hq, Hkv, S, D, int(window), _ptr(workspace), wbytes, dt,
          _stream(stream))
    return dq, dk, dv, dsink
