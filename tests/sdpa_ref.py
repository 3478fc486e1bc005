"""Library-based references used to pin the oracle (CPU, float64).

These express the method through ``torch.nn.functional.scaled_dot_product_attention``
and ``torch.logsumexp`` instead of the oracle's own loops:

* grouped-query attention becomes plain multi-head attention after
  ``repeat_interleave`` of the KV heads;
* the sink becomes one extra *virtual* key whose logit is s_h (a zero key
  plus an additive bias of s_h) and whose value vector is zero -- the
  reading of the "MiMo-V2-Flash Technical Report" digest, 前置知识 /
  注意力sink偏置, where attention mass can go to a virtual sink token
  instead of a real token.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def sdpa_with_sink(q, k, v, sink, allowed):
    """q [B, Sq, Hq, D], k/v [B, Skv, Hkv, D], sink [Hq] (may hold -inf),
    allowed: bool [B, Sq, Skv] (or broadcastable) -- key j visible to query i.

    Returns out [B, Sq, Hq, D] and lse [B, Hq, Sq] as float64 numpy arrays.
    """
    q = torch.as_tensor(np.asarray(q, dtype=np.float64))
    k = torch.as_tensor(np.asarray(k, dtype=np.float64))
    v = torch.as_tensor(np.asarray(v, dtype=np.float64))
    sink = torch.as_tensor(np.asarray(sink, dtype=np.float64))
    allowed = torch.as_tensor(np.asarray(allowed, dtype=bool))
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qh = q.permute(0, 2, 1, 3)                                        # B Hq Sq D
    kh = k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)            # B Hq Skv D
    vh = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    zero = torch.zeros(B, Hq, 1, D, dtype=torch.float64)
    kh = torch.cat([kh, zero], dim=2).contiguous()                    # virtual key
    vh = torch.cat([vh, zero], dim=2).contiguous()                    # value 0
    allowed = allowed.expand(B, Sq, Skv)
    bias = torch.full((B, Hq, Sq, Skv + 1), -math.inf, dtype=torch.float64)
    bias[..., :Skv] = torch.where(allowed[:, None], 0.0, -math.inf)
    bias[..., Skv] = sink[None, :, None]
    scale = 1.0 / math.sqrt(D)
    out = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=bias, scale=scale)
    logits = torch.matmul(qh, kh.transpose(-1, -2).contiguous()) * scale + bias
    lse = torch.logsumexp(logits, dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy()


def band_mask(S: int, W: int):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    return (j <= i) & (j > i - W)


def causal_bottom_right(Sq: int, Skv: int):
    i = np.arange(Sq)[:, None] + (Skv - Sq)
    j = np.arange(Skv)[None, :]
    return j <= i
