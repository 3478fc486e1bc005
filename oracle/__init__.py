"""fp64 CPU oracle for sliding-window attention with a learnable sink.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The product package never
imports it, and it imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (plain loops, double precision, OpenMP
over rows and heads).  This module only builds that file with gcc, turns
numpy arrays into contiguous float64 buffers, and states each call's key set:

* sliding-window prefill -- row i sees positions max(0, i-W+1) .. i
  ("MiMo-V2-Flash Technical Report" digest, 前置知识 / 混合注意力机制 and
  核心方法: a 128-token local window);
* global causal attention -- with S_q queries at the end of S_kv keys, row i
  sits at position S_kv - S_q + i and sees 0 .. that position (same digest,
  混合注意力机制: global layers see the whole sequence);
* packed batches of sequences of different lengths -- see ``prefill_varlen``;
* ring decode -- see ``ring_decode``;
* the gradients of the first two -- see ``attend_backward``;
* block maxima of the global layer's logits -- see ``block_max``.

The sink term is described in the same digest, 前置知识 / 注意力sink偏置.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def bind(path: str):
    """Load a compiled oracle library from ``path`` and declare its C
    signatures (tests also load deliberately broken copies this way)."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.oracle_attend_rows.argtypes = [dp, ip, ip, ip, dp, dp, dp, dp, dp,
                                       i64, i64, i64, i64, i64]
    lib.oracle_attend_rows.restype = None
    lib.oracle_ring_decode.argtypes = [dp, dp, dp, dp, ip, dp, dp,
                                       i64, i64, i64, i64, i64, i64, i64]
    lib.oracle_ring_decode.restype = None
    lib.oracle_attend_backward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                           i64, i64, i64, i64, i64, i64]
    lib.oracle_attend_backward.restype = None
    lib.oracle_rope.argtypes = [dp, ip, dp, i64, i64, i64, ctypes.c_double]
    lib.oracle_rope.restype = None
    lib.oracle_block_max.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, i64, i64]
    lib.oracle_block_max.restype = None
    lib.oracle_count_window_pairs.argtypes = [i64, i64]
    lib.oracle_count_window_pairs.restype = i64
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = bind(_LIB)
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def attend_rows(q_rows, row_batch, lo, hi, k, v, sink):
    """Rows r of ``q_rows`` [R, Hq, D] (batch ``row_batch[r]``) over key
    positions lo[r]..hi[r] of ``k``/``v`` [B, N, Hkv, D].

    Returns (out [R, Hq, D], lse [R, Hq]) in float64.
    """
    q_rows, k, v, sink = _f64(q_rows), _f64(k), _f64(v), _f64(sink)
    row_batch, lo, hi = _i64(row_batch), _i64(lo), _i64(hi)
    R, Hq, D = q_rows.shape
    B, N, Hkv, Dk = k.shape
    assert Dk == D and v.shape == k.shape and sink.shape == (Hq,)
    assert Hq % Hkv == 0 and row_batch.shape == lo.shape == hi.shape == (R,)
    assert R == 0 or (row_batch.min() >= 0 and row_batch.max() < B)
    out = np.zeros((R, Hq, D), dtype=np.float64)
    lse = np.zeros((R, Hq), dtype=np.float64)
    if R:
        _load().oracle_attend_rows(_dp(q_rows), _ip(row_batch), _ip(lo), _ip(hi),
                                   _dp(k), _dp(v), _dp(sink), _dp(out), _dp(lse),
                                   R, N, Hq, Hkv, D)
    return out, lse


def swa_prefill_rows(q_rows, row_batch, row_pos, k, v, sink, window):
    """Sampled rows of a causal sliding-window prefill: row r is the query at
    position ``row_pos[r]`` of sequence ``row_batch[r]``."""
    row_pos = _i64(row_pos)
    lo = np.maximum(0, row_pos - int(window) + 1)
    return attend_rows(q_rows, row_batch, lo, row_pos, k, v, sink)


def swa_prefill(q, k, v, sink, window):
    """Full causal sliding-window prefill.

    q [B, S, Hq, D], k/v [B, S, Hkv, D], sink [Hq]
    -> out [B, S, Hq, D], lse [B, Hq, S] (float64).
    """
    q = _f64(q)
    B, S, Hq, D = q.shape
    rb = np.repeat(np.arange(B), S)
    rp = np.tile(np.arange(S), B)
    out, lse = swa_prefill_rows(q.reshape(B * S, Hq, D), rb, rp, k, v, sink, window)
    return out.reshape(B, S, Hq, D), lse.reshape(B, S, Hq).transpose(0, 2, 1).copy()


def prefill_varlen(q, k, v, sink, cu_seqlens, window):
    """Packed batch of sequences of different lengths: sequence b is rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1 of q [total, Hq, D] and k/v
    [total, Hkv, D], and is a causal window-``window`` prefill on its own
    (positions restart at 0 per sequence; no row sees another sequence).
    Serving mixed context lengths together: "小米罗福莉：MiMo-V2.5如何做到
    又快又强又便宜？| ICML 2026", §06 Q&A, audience E.

    -> out [total, Hq, D], lse [Hq, total] (float64).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    total, Hq, D = q.shape
    assert cu[0] == 0 and cu[-1] == total and all(a <= b for a, b in zip(cu, cu[1:]))
    out = np.zeros((total, Hq, D), dtype=np.float64)
    lse = np.zeros((Hq, total), dtype=np.float64)
    for s0, s1 in zip(cu, cu[1:]):
        if s1 == s0:
            continue
        o, l = swa_prefill(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], sink, window)
        out[s0:s1] = o[0]
        lse[:, s0:s1] = l[0]
    return out, lse


def global_rows(q_rows, row_batch, row_pos, k, v, sink):
    """Sampled rows of global causal attention: row r is the query at absolute
    position ``row_pos[r]`` and sees keys 0 .. row_pos[r]."""
    row_pos = _i64(row_pos)
    return attend_rows(q_rows, row_batch, np.zeros_like(row_pos), row_pos, k, v, sink)


def global_attn(q, k, v, sink):
    """Global causal attention with the queries aligned to the end of the keys.

    q [B, S_q, Hq, D], k/v [B, S_kv, Hkv, D] with S_q <= S_kv, sink [Hq]
    -> out [B, S_q, Hq, D], lse [B, Hq, S_q] (float64).
    """
    q = _f64(q)
    B, Sq, Hq, D = q.shape
    Skv = np.asarray(k).shape[1]
    assert Sq <= Skv
    rb = np.repeat(np.arange(B), Sq)
    rp = np.tile(np.arange(Skv - Sq, Skv), B)
    out, lse = global_rows(q.reshape(B * Sq, Hq, D), rb, rp, k, v, sink)
    return out.reshape(B, Sq, Hq, D), lse.reshape(B, Sq, Hq).transpose(0, 2, 1).copy()


def ring_decode(q, kcache, vcache, sink, cache_len=None, window=None):
    """Decode T new query tokens per sequence against a W-slot ring cache.

    q [B, T, Hq, D]; kcache/vcache [B, Hkv, W, D] with the key of absolute
    position P in slot P mod W; cache_len [B] = tokens written so far
    including the T new ones (None: every ring is exactly full, L = W);
    window = keys per query (default W, at most W).  Query t is at position
    p = L - T + t and sees positions max(0, L-W, p-window+1) .. p.
    Returns out [B, T, Hq, D], lse [B, T, Hq] (float64).
    """
    q, kcache, vcache, sink = _f64(q), _f64(kcache), _f64(vcache), _f64(sink)
    B, T, Hq, D = q.shape
    Bk, Hkv, W, Dk = kcache.shape
    assert Bk == B and Dk == D and vcache.shape == kcache.shape and Hq % Hkv == 0
    cl = _i64(np.full(B, W) if cache_len is None else cache_len)
    assert cl.shape == (B,)
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    lse = np.zeros((B, T, Hq), dtype=np.float64)
    wnd = W if window is None else int(window)
    assert 1 <= wnd <= W
    _load().oracle_ring_decode(_dp(q), _dp(kcache), _dp(vcache), _dp(sink), _ip(cl),
                               _dp(out), _dp(lse), B, T, Hq, Hkv, W, D, wnd)
    return out, lse


def rope(x, pos, theta):
    """Rotary position embedding of x [n, H, D] at absolute positions pos [n]
    (dimension i paired with i + D/2, angle pos * theta^(-2i/D))."""
    x = _f64(x)
    n, H, D = x.shape
    pos = _i64(pos)
    assert pos.shape == (n,) and D % 2 == 0
    y = np.empty_like(x)
    _load().oracle_rope(_dp(x), _ip(pos), _dp(y), n, H, D, float(theta))
    return y


def rope_append(q, k_new, v_new, kcache, vcache, cache_len_old, theta):
    """One decode step's preparation: RoPE on the T new queries and keys at
    positions L_old + t, and the keys (rotated) and values written to ring
    slots (L_old + t) mod W.  q [B, T, Hq, D]; k_new, v_new [B, T, Hkv, D];
    kcache, vcache [B, Hkv, W, D] (copies are updated and returned);
    cache_len_old [B] = tokens in the cache before the step.
    Returns (q_rot, kcache, vcache)."""
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    kc, vc = _f64(kcache).copy(), _f64(vcache).copy()
    B, T, Hq, D = q.shape
    Hkv, W = kc.shape[1], kc.shape[2]
    lo = _i64(cache_len_old)
    pos = (lo[:, None] + np.arange(T)[None, :]).reshape(-1)
    q_rot = rope(q.reshape(B * T, Hq, D), pos, theta).reshape(B, T, Hq, D)
    k_rot = rope(k_new.reshape(B * T, Hkv, D), pos, theta).reshape(B, T, Hkv, D)
    for b in range(B):
        for t in range(T):
            slot = (int(lo[b]) + t) % W
            kc[b, :, slot] = k_rot[b, t]
            vc[b, :, slot] = v_new[b, t]
    return q_rot, kc, vc


def attend_backward(q, k, v, sink, dout, window, lib=None):
    """Gradients of causal sliding-window attention with a sink (window >= S:
    global causal attention) for the upstream gradient ``dout``.

    q, dout [B, S, Hq, D]; k, v [B, S, Hkv, D]; sink [Hq]
    -> dq [B, S, Hq, D], dk, dv [B, S, Hkv, D], dsink [Hq] (float64; dsink
    summed over the batch).  ``lib`` lets tests run a modified copy."""
    q, k, v, sink, dout = _f64(q), _f64(k), _f64(v), _f64(sink), _f64(dout)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dsink = np.empty(Hq)
    (lib or _load()).oracle_attend_backward(
        _dp(q), _dp(k), _dp(v), _dp(sink), _dp(dout), _dp(dq), _dp(dk), _dp(dv), _dp(dsink),
        B, S, Hq, Hkv, D, int(min(window, S)))
    return dq, dk, dv, dsink


def block_max(q, k, block_k, lib=None):
    """Largest scaled logit q_i . k_j / sqrt(D) over the visible pairs of each
    (32-row query block, block_k-key block) of global causal attention with
    the queries at the end of the keys; -inf for blocks with no visible pair.

    q [B, S_q, Hq, D], k [B, S_kv, Hkv, D]
    -> [B, Hq, ceil(S_q / 32), ceil(S_kv / block_k)] (float64)."""
    q, k = _f64(q), _f64(k)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    assert Sq <= Skv and Hq % Hkv == 0 and block_k >= 1
    out = np.empty((B, Hq, (Sq + 31) // 32, (Skv + block_k - 1) // block_k))
    (lib or _load()).oracle_block_max(_dp(q), _dp(k), _dp(out), B, Sq, Skv, Hq, Hkv, D,
                                      int(block_k))
    return out


def count_window_pairs(S: int, W: int) -> int:
    """(query, key) pairs of one causal window-W layer over S tokens, counted
    row by row."""
    return int(_load().oracle_count_window_pairs(int(S), int(W)))


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads for the oracle's later parallel loops (timing runs only)."""
    _load().oracle_set_threads(int(n))
