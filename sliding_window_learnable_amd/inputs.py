"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws Gaussian tensors of
the workload shapes from explicitly seeded generators, so that the HIP path
and the CPU oracle see identical values.

Seed recipe: ``1000*config + 10*layer + {q: 1, k: 2, v: 3, sink: 4, dout: 5}``
(dout: the upstream gradient of a backward pass), with
the workload configs numbered 1..5 (tiny reference, 32K prefill, batched
decode, hybrid 5:1 stack, long context).  Values are drawn in float32 with
``torch.randn`` and rounded to bfloat16 (round-to-nearest-even) when the
workload is bfloat16.  The sink is always float32, one value per query head.
"""
from __future__ import annotations

import torch

TENSOR_SEED = {"q": 1, "k": 2, "v": 3, "sink": 4, "dout": 5}


def seed_for(config: int, layer: int, tensor: str) -> int:
    return 1000 * int(config) + 10 * int(layer) + TENSOR_SEED[tensor]


def randn(shape, seed: int, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """N(0, 1) samples of ``shape`` from a generator seeded with ``seed`` on
    ``device``, drawn in float32 and then cast to ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def attention_inputs(config: int, layer: int, B: int, S_q: int, S_kv: int, Hq: int,
                     Hkv: int, D: int, dtype=torch.bfloat16, device="cpu"):
    """q [B, S_q, Hq, D], k and v [B, S_kv, Hkv, D] in ``dtype``, sink [Hq] float32."""
    q = randn((B, S_q, Hq, D), seed_for(config, layer, "q"), dtype, device)
    k = randn((B, S_kv, Hkv, D), seed_for(config, layer, "k"), dtype, device)
    v = randn((B, S_kv, Hkv, D), seed_for(config, layer, "v"), dtype, device)
    sink = randn((Hq,), seed_for(config, layer, "sink"), torch.float32, device)
    return q, k, v, sink


def upstream_grad(config: int, layer: int, B: int, S: int, Hq: int, D: int,
                  dtype=torch.bfloat16, device="cpu"):
    """dout [B, S, Hq, D] in ``dtype``: the gradient arriving at the attention output."""
    return randn((B, S, Hq, D), seed_for(config, layer, "dout"), dtype, device)


def ring_inputs(config: int, layer: int, B: int, T: int, Hq: int, Hkv: int, W: int,
                D: int, dtype=torch.bfloat16, device="cpu"):
    """q [B, T, Hq, D], kcache and vcache [B, Hkv, W, D] in ``dtype``, sink [Hq]."""
    q = randn((B, T, Hq, D), seed_for(config, layer, "q"), dtype, device)
    kc = randn((B, Hkv, W, D), seed_for(config, layer, "k"), dtype, device)
    vc = randn((B, Hkv, W, D), seed_for(config, layer, "v"), dtype, device)
    sink = randn((Hq,), seed_for(config, layer, "sink"), torch.float32, device)
    return q, kc, vc, sink


def cache_lengths(B: int, low: int, high: int, seed: int) -> torch.Tensor:
    """int32 [B] lengths uniform in [low, high] (inclusive) from ``seed``."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    return torch.randint(int(low), int(high) + 1, (B,), generator=gen, dtype=torch.int32)


def packed_inputs(config: int, layer: int, lengths, Hq: int, Hkv: int, D: int,
                  dtype=torch.bfloat16, device="cpu"):
    """A packed batch of sequences of the given lengths: q [total, Hq, D],
    k and v [total, Hkv, D] in ``dtype``, sink [Hq] float32 and cu_seqlens
    int32 [B + 1] (row offsets of the sequences)."""
    lengths = [int(n) for n in lengths]
    total = sum(lengths)
    q = randn((total, Hq, D), seed_for(config, layer, "q"), dtype, device)
    k = randn((total, Hkv, D), seed_for(config, layer, "k"), dtype, device)
    v = randn((total, Hkv, D), seed_for(config, layer, "v"), dtype, device)
    sink = randn((Hq,), seed_for(config, layer, "sink"), torch.float32, device)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return q, k, v, sink, cu.to(device)
