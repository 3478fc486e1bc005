"""Algorithmic FLOP and byte counts of each call, for throughput and roofline
reporting.

Counting rules:
* flops = 4 * D per (query row, query head, attended key): 2D for q.k and
  2D for p*v.  Masked or padded work, the softmax and the exponentials are
  not counted.
* bytes = every input and output tensor crossing HBM exactly once (q, k, v
  or the ring caches, out, lse); halo re-reads and split-KV workspace
  traffic are not counted.

Key counts follow the call semantics: a causal window-W layer over S tokens
attends W*S - W*(W-1)/2 pairs when S >= W (every row sees min(i+1, W) keys);
a global causal layer attends S*(S+1)/2.
"""
from __future__ import annotations

BF16, F32 = 2, 4

# MI355X published peaks (dense, no sparsity)
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2516.6
PEAK_F32_MFMA_TFLOPS = 157.3


def roofline_frac(flops: float, nbytes: float, seconds: float) -> float:
    """Achieved flops over the roofline min(bf16 MFMA peak, AI * HBM peak),
    AI = flops / bytes (algorithmic)."""
    roof = min(PEAK_BF16_TFLOPS * 1e12, flops / nbytes * PEAK_HBM_GBS * 1e9)
    return flops / seconds / roof


def window_pairs(S: int, W: int) -> int:
    """(row, key) pairs of a causal window-W layer over S tokens."""
    m = min(S, W)
    return m * (m + 1) // 2 + max(0, S - W) * W


def causal_pairs(S_q: int, S_kv: int) -> int:
    """(row, key) pairs of global causal attention with S_q queries aligned to
    the end of S_kv keys: row i sees S_kv - S_q + i + 1 keys."""
    first = S_kv - S_q + 1
    return S_q * first + S_q * (S_q - 1) // 2


def ring_pairs(T: int, W: int, L: int) -> int:
    """Pairs of one ring-decode sequence with L tokens written (T new)."""
    oldest = max(0, L - W)
    return sum(max(0, (L - T + t) - oldest + 1) for t in range(T))


def prefill_flops(B, S, Hq, D, W) -> int:
    return 4 * D * Hq * B * window_pairs(S, W)


def prefill_bytes(B, S, Hq, Hkv, D, elt=BF16, with_lse=True) -> int:
    qo = 2 * B * S * Hq * D * elt
    kv = 2 * B * S * Hkv * D * elt
    return qo + kv + (B * Hq * S * F32 if with_lse else 0)


def global_flops(B, S_q, S_kv, Hq, D) -> int:
    return 4 * D * Hq * B * causal_pairs(S_q, S_kv)


def global_bytes(B, S_q, S_kv, Hq, Hkv, D, elt=BF16, with_lse=True) -> int:
    qo = 2 * B * S_q * Hq * D * elt
    kv = 2 * B * S_kv * Hkv * D * elt
    return qo + kv + (B * Hq * S_q * F32 if with_lse else 0)


def backward_flops(B, S, Hq, D, W) -> int:
    """Attention backward: 10 * D per attended (row, head, key) pair -- the
    recomputed q.k (2D) and dO.v (2D), and dv, dk, dq (2D each)."""
    return 10 * D * Hq * B * window_pairs(S, W)


def backward_bytes(B, S, Hq, Hkv, D, elt=BF16) -> int:
    """q, k, v, out, dout, lse read once; dq, dk, dv written once."""
    q_like = 4 * B * S * Hq * D * elt          # q, out, dout read; dq written
    kv_like = 4 * B * S * Hkv * D * elt        # k, v read; dk, dv written
    return q_like + kv_like + B * Hq * S * F32


def decode_flops(B, T, Hq, D, W, L=None) -> int:
    L = W if L is None else L
    return 4 * D * Hq * B * ring_pairs(T, W, L)


def decode_bytes(B, T, Hq, Hkv, W, D, elt=BF16, with_lse=True) -> int:
    qo = 2 * B * T * Hq * D * elt
    kv = 2 * B * Hkv * W * D * elt
    return qo + kv + (B * Hq * T * F32 if with_lse else 0)


def hybrid_ratios(S: int, W: int, n_swa: int):
    """Full attention in every layer vs n_swa window-W layers + 1 global layer:
    (attention-compute reduction, KV-cache reduction)."""
    ga = causal_pairs(S, S)
    sw = window_pairs(S, W)
    layers = n_swa + 1
    compute = layers * ga / (n_swa * sw + ga)
    kv = layers * S / (n_swa * min(S, W) + S)
    return compute, kv
