#!/usr/bin/env python3
"""Benchmark of the sliding-window + sink attention hot path on one MI355X.

Headline (one JSON line on stdout): swa_sink_prefill on the 32K prefill
workload -- B=1, S=32768, Hq=64, Hkv=8, D=128, window 128, bf16 inputs,
fp32 accumulation, bf16 out + fp32 LSE -- in algorithmic TFLOP/s.  One
"step" is one prefill call over the whole workload.  Alongside it, in the
same JSON object:
  roofline      the prefill kernel against HBM bandwidth (its bound)
  cpu_baseline  the fp64 oracle timed on the host cores over the same workload
  decode        ring-cache decode, B=256, 128 slots, T_q = 1 and 4, in HBM GB/s
  hybrid_5to1   5 SWA layers + 1 global layer at S=65536: per-layer-type time
  long_context  SWA prefill at S=262144; global decode B=8 over 262144 keys
  backward      swa_sink_backward (dq, dk, dv, dsink) at the 32K SWA workload
                and on a 16K global layer, with the forward time beside it
  varlen        packed prefill of 16 sequences of mixed length (one context
                bucket), window 128 and global, against the padded batch
  oracle_by_config  the fp64 oracle beside the GPU on every configuration above
                (full or stated samples): time, GFLOP/s, speed-up, max |error|
Inputs are seeded synthetic Gaussian tensors resident in HBM before timing.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only SECTION]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SWA+sink attention TFLOP/s (prefill, % MFMA peak) and decode HBM GB/s, 1 GPU"
PREFILL_KERNEL_SRC = os.path.join(ROOT, "sliding_window_learnable_amd", "csrc", "swa_prefill.hip")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "swa_prefill_32k_hbm_traffic.md")


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The shader clock needs ~100 prefill calls (~40 ms) to reach its
    # sustained value: warm up past that before timing.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=150)
    # Before the warm-up steps of each timed section, the GPU is kept busy with
    # the same call for this long: from idle the shader clock takes ~40 ms of
    # sustained load to reach its steady value, longer than a few warm-up
    # steps last.  Not part of the timed region.
    ap.add_argument("--settle-ms", type=float, default=300.0)
    ap.add_argument("--only", default="all",
                    choices=["all", "prefill", "decode", "hybrid", "long", "backward", "varlen",
                             "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--oracle-ga-stride", type=int, default=256,
                    help="query-row stride of the oracle's sample of the 64K global layer")
    return ap.parse_args()


SETTLE_S = 0.3


def settle(fn):
    """Keeps the GPU busy with fn for SETTLE_S seconds (untimed) so the shader
    clock reaches its sustained value; returns the number of calls made."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(8):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def timed(fn, steps, warmup):
    """Average ms per call of fn(i) over `steps` back-to-back calls, timed with
    HIP events on the stream the kernels are launched on (torch's current
    stream, which the binding passes to the C ABI).  The clock is settled
    first, then `warmup` untimed calls precede the timed ones."""
    import torch
    stream = torch.cuda.current_stream()
    settle(fn)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(i)
    t1.record(stream)
    t1.synchronize()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def per_call(fn, batches, size):
    """Median, p10 and p90 of the per-call time (us) over `batches` batches of
    `size` back-to-back calls, each batch bracketed by HIP events on the
    launch stream (an event between every call would add a gap per call and
    change what is measured).  Run right after `timed`, with the clock warm."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for j in range(batches):
        for i in range(size):
            fn(j * size + i)
        ev[j + 1].record(stream)
    ev[batches].synchronize()
    us = sorted(ev[j].elapsed_time(ev[j + 1]) * 1e3 / size for j in range(batches))
    pick = lambda f: us[min(batches - 1, int(round(f * (batches - 1))))]
    return {"median_us": pick(0.5), "p10_us": pick(0.1), "p90_us": pick(0.9),
            "batches": batches, "calls_per_batch": size}


def sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_record():
    """HBM bytes per prefill launch from the committed rocprofv3 counter
    summary, or None when missing or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_RECORD):
        return None
    text = open(TRAFFIC_RECORD).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sha256(PREFILL_KERNEL_SRC):
        return None
    return float(m_b.group(1))


# --------------------------------------------------------------------------- sections

def bench_prefill(args, swa, acc, torch):
    from sliding_window_learnable_amd import inputs
    B, S, Hq, Hkv, D, W = 1, 32768, 64, 8, 128, 128
    q, k, v, sink = inputs.attention_inputs(2, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
    log("prefill 32K: warmup %d, steps %d" % (args.warmup, args.steps))
    ms = timed(lambda i: swa.swa_sink_prefill(q, k, v, sink, W, out=out, lse=lse),
               args.steps, args.warmup)
    flops = acc.prefill_flops(B, S, Hq, D, W)
    nbytes = acc.prefill_bytes(B, S, Hq, Hkv, D)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    dist = per_call(lambda i: swa.swa_sink_prefill(q, k, v, sink, W, out=out, lse=lse), 20, 10)
    res = dict(ms=ms, per_call=dist, tflops=tflops, gbs=gbs, flops=flops, bytes=nbytes,
               cache="one input set: its 1.2 GB of inputs and outputs exceed the 256 MB "
                     "Infinity Cache",
               tokens_per_s=B * S / (ms * 1e-3),
               frac_mfma_peak=tflops / acc.PEAK_BF16_TFLOPS,
               frac_hbm_peak=gbs / acc.PEAK_HBM_GBS,
               frac_roofline=acc.roofline_frac(flops, nbytes, ms * 1e-3))
    res["tensors"] = (q, k, v, sink, out)
    return res


def bench_cpu_baseline(args, acc, torch, tensors):
    """The fp64 oracle, as it stands, on the host cores: whole passes over the
    32K prefill workload (every row, every head), repeated until about
    --cpu-seconds of CPU time has been spent."""
    import numpy as np
    import oracle
    q, k, v, sink, gpu_out = tensors
    B, S, Hq, D = q.shape
    W = 128
    q64 = q.double().cpu().numpy()
    k64 = k.double().cpu().numpy()
    v64 = v.double().cpu().numpy()
    s64 = sink.double().cpu().numpy()
    t = time.perf_counter()
    ref, _ = oracle.swa_prefill(q64, k64, v64, s64, W)
    first = time.perf_counter() - t
    err = float(np.abs(gpu_out.double().cpu().numpy() - ref).max())
    del ref
    reps = int(max(1, min(20, round(args.cpu_seconds / max(first, 1e-6)))))
    log("cpu baseline: one pass %.2fs, %d passes" % (first, reps))
    t = time.perf_counter()
    for _ in range(reps):
        oracle.swa_prefill(q64, k64, v64, s64, W)
    dt = time.perf_counter() - t
    flops = reps * acc.prefill_flops(B, S, Hq, D, W)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "max_abs_err_vs_gpu": err,
            "sample": "%d full pass(es) of the 32K prefill workload (all 32768 rows, 64 heads), "
                      "fp64, %.1f s total" % (reps, dt),
            "seconds": dt}


def bench_decode(args, swa, acc, torch):
    from sliding_window_learnable_amd import inputs
    B, Hq, Hkv, D, W = 256, 64, 8, 128, 128
    nsets = 5          # 5 x 128 MiB of ring caches > 256 MiB Infinity Cache
    res = {"workload": "swa_sink_decode B=256 Hq=64 Hkv=8 D=128 ring=128 bf16, full rings",
           "cache_rotation": "%d independent input sets (%d MiB of KV) cycled per call"
                             % (nsets, nsets * 128)}
    for T in (1, 4):
        sets = [inputs.ring_inputs(3, layer, B, T, Hq, Hkv, W, D, torch.bfloat16, "cuda")
                for layer in range(nsets)]
        outs = [torch.empty_like(s[0]) for s in sets]
        lses = [torch.empty((B, Hq, T), device="cuda", dtype=torch.float32) for _ in sets]

        def call(i):
            s = sets[i % nsets]
            swa.swa_sink_decode(s[0], s[1], s[2], s[3], out=outs[i % nsets], lse=lses[i % nsets])

        steps = max(200, 10 * args.steps)
        log("decode T_q=%d: %d calls" % (T, steps))
        ms = timed(call, steps, 200)
        dist = per_call(call, 20, 50)
        nbytes = acc.decode_bytes(B, T, Hq, Hkv, W, D)
        flops = acc.decode_flops(B, T, Hq, D, W)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res["T_q=%d" % T] = dict(us_per_call=ms * 1e3, per_call=dist, hbm_gbs=gbs,
                                 frac_hbm_peak=gbs / acc.PEAK_HBM_GBS,
                                 frac_roofline=acc.roofline_frac(flops, nbytes, ms * 1e-3),
                                 tflops=flops / (ms * 1e-3) / 1e12,
                                 tokens_per_s=B * T / (ms * 1e-3), bytes=nbytes)
        del sets, outs, lses
        torch.cuda.empty_cache()
    res["time_ratio_T4_over_T1"] = res["T_q=4"]["us_per_call"] / res["T_q=1"]["us_per_call"]

    # MTP with rollback: RoPE + ring append of 1 + 3 tokens, then decode in
    # rings of W + T - 1 = 131 slots (every draft sees its full window).
    T, R = 4, W + 3
    sets = [inputs.ring_inputs(3, 10 + layer, B, T, Hq, Hkv, R, D, torch.bfloat16, "cuda")
            for layer in range(nsets)]
    news = [(inputs.ring_inputs(3, 20 + layer, B, T, Hq, Hkv, 1, D, torch.bfloat16, "cuda")[0],
             torch.randn((B, T, Hkv, D), device="cuda").to(torch.bfloat16),
             torch.randn((B, T, Hkv, D), device="cuda").to(torch.bfloat16)) for layer in range(nsets)]
    lens_old = inputs.cache_lengths(B, R, 1 << 20, 33).to("cuda")
    lens = lens_old + T
    qrot = [torch.empty_like(n[0]) for n in news]
    outs = [torch.empty_like(n[0]) for n in news]

    def append(i):
        s_, n_ = sets[i % nsets], news[i % nsets]
        swa.swa_sink_rope_append(n_[0], n_[1], n_[2], s_[1], s_[2], lens_old, 1e6,
                                 q_rot=qrot[i % nsets])

    def decode_ring(i):
        s_ = sets[i % nsets]
        swa.swa_sink_decode_ring(qrot[i % nsets], s_[1], s_[2], s_[3], W, lens,
                                 out=outs[i % nsets], want_lse=False)

    steps = max(200, 10 * args.steps)
    log("rollback ring: append + decode, %d calls each" % steps)
    ms_a = timed(append, steps, 200)
    ms_d = timed(decode_ring, steps, 200)
    nbytes = acc.decode_bytes(B, T, Hq, Hkv, R, D)
    res["rollback_ring_T_q=4"] = dict(
        ring_slots=R, window=W, append_us=ms_a * 1e3, decode_us=ms_d * 1e3,
        decode_hbm_gbs=nbytes / (ms_d * 1e-3) / 1e9,
        decode_frac_hbm_peak=nbytes / (ms_d * 1e-3) / 1e9 / acc.PEAK_HBM_GBS,
        step_us=(ms_a + ms_d) * 1e3)
    del sets, news, qrot, outs
    torch.cuda.empty_cache()
    return res


def bench_hybrid(args, swa, acc, torch):
    """5 SWA+sink layers (window 128) then 1 global causal+sink layer, S=65536."""
    from sliding_window_learnable_amd import inputs
    B, S, Hq, Hkv, D, W = 1, 65536, 64, 8, 128, 128
    layers = [inputs.attention_inputs(4, layer, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
              for layer in range(6)]
    out = torch.empty_like(layers[0][0])
    lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)

    def swa_layers(i):
        for q, k, v, s in layers[:5]:
            swa.swa_sink_prefill(q, k, v, s, W, out=out, lse=lse)

    def ga_layer(i):
        q, k, v, s = layers[5]
        swa.global_sink_attn(q, k, v, s, out=out, lse=lse)

    q5, k5, v5, s5 = layers[5]
    bmax = torch.empty((B, Hq, S // 32, S // 128), device="cuda", dtype=torch.float32)

    def ga_layer_blocks(i):
        swa.global_sink_attn_block_max(q5, k5, v5, s5, block_k=128, out=out, lse=lse,
                                       block_max=bmax)

    log("hybrid 5:1 at S=65536")
    ms_swa5 = timed(swa_layers, 5, 1)
    ms_ga = timed(ga_layer, 3, 1)
    ms_ga_blk = timed(ga_layer_blocks, 3, 1)
    f_swa = acc.prefill_flops(B, S, Hq, D, W)
    f_ga = acc.global_flops(B, S, S, Hq, D)
    compute_red, kv_red = acc.hybrid_ratios(S, W, 5)
    compute_red7, kv_red7 = acc.hybrid_ratios(S, W, 7)
    del layers, q5, k5, v5, s5, bmax
    torch.cuda.empty_cache()
    return {
        "workload": "5 x swa_sink_prefill (window 128) + 1 x global_sink_attn, B=1 S=65536 "
                    "Hq=64 Hkv=8 D=128 bf16, seeds per layer",
        "swa_layer_ms": ms_swa5 / 5, "global_layer_ms": ms_ga, "stack_ms": ms_swa5 + ms_ga,
        "swa_layer_tflops": f_swa / (ms_swa5 / 5 * 1e-3) / 1e12,
        "global_layer_tflops": f_ga / (ms_ga * 1e-3) / 1e12,
        "global_layer_frac_mfma_peak": f_ga / (ms_ga * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS,
        "global_layer_frac_roofline": acc.roofline_frac(
            f_ga, acc.global_bytes(B, S, S, Hq, Hkv, D), ms_ga * 1e-3),
        "swa_layer_frac_roofline": acc.roofline_frac(
            f_swa, acc.prefill_bytes(B, S, Hq, Hkv, D), ms_swa5 / 5 * 1e-3),
        "swa_layer_hbm_gbs": acc.prefill_bytes(B, S, Hq, Hkv, D) / (ms_swa5 / 5 * 1e-3) / 1e9,
        "flop_ratio_swa_over_global_per_layer": f_swa / f_ga,
        "flop_share_of_5_swa_layers": 5 * f_swa / (5 * f_swa + f_ga),
        "attention_compute_reduction_vs_6_global": compute_red,
        "kv_cache_reduction_vs_6_global": kv_red,
        "measured_time_reduction_vs_6_global": 6 * ms_ga / (ms_swa5 + ms_ga),
        # the global layer with the block-score side output (32-row x 128-key blocks)
        "global_layer_with_block_max_ms": ms_ga_blk,
        "block_max_overhead": ms_ga_blk / ms_ga - 1.0,
        # 7:1 schedule (Pro): the same two layer types, 7 SWA layers per global one
        "schedule_7to1": {
            "stack_ms": 7 * ms_swa5 / 5 + ms_ga,
            "attention_compute_reduction_vs_8_global": compute_red7,
            "kv_cache_reduction_vs_8_global": kv_red7,
            "measured_time_reduction_vs_8_global": 8 * ms_ga / (7 * ms_swa5 / 5 + ms_ga),
        },
    }


def bench_long(args, swa, acc, torch):
    from sliding_window_learnable_amd import inputs
    res = {}
    B, S, Hq, Hkv, D, W = 1, 262144, 64, 8, 128, 128
    q, k, v, sink = inputs.attention_inputs(5, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
    log("long context: SWA prefill S=262144")
    ms = timed(lambda i: swa.swa_sink_prefill(q, k, v, sink, W, out=out, lse=lse), 5, 2)
    f = acc.prefill_flops(B, S, Hq, D, W)
    nb = acc.prefill_bytes(B, S, Hq, Hkv, D)
    res["swa_prefill_262144"] = dict(ms=ms, tflops=f / (ms * 1e-3) / 1e12,
                                     hbm_gbs=nb / (ms * 1e-3) / 1e9,
                                     frac_hbm_peak=nb / (ms * 1e-3) / 1e9 / acc.PEAK_HBM_GBS,
                                     frac_roofline=acc.roofline_frac(f, nb, ms * 1e-3),
                                     tokens_per_s=S / (ms * 1e-3))
    del q, k, v, out, lse
    torch.cuda.empty_cache()

    B, Sq, Skv = 8, 1, 262144
    q, k, v, sink = inputs.attention_inputs(5, 1, B, Sq, Skv, Hq, Hkv, D, torch.bfloat16, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), device="cuda", dtype=torch.float32)
    ws = torch.empty(swa.global_sink_attn_workspace_bytes(B, Hq, Hkv, Sq, Skv, D),
                     device="cuda", dtype=torch.uint8)
    log("long context: global decode B=8 over 262144 keys")
    ms = timed(lambda i: swa.global_sink_attn(q, k, v, sink, out=out, lse=lse, workspace=ws), 20, 3)
    nb = acc.global_bytes(B, Sq, Skv, Hq, Hkv, D)
    res["global_decode_B8_262144"] = dict(
        ms=ms, hbm_gbs=nb / (ms * 1e-3) / 1e9, frac_hbm_peak=nb / (ms * 1e-3) / 1e9 / acc.PEAK_HBM_GBS,
        frac_roofline=acc.roofline_frac(acc.global_flops(B, Sq, Skv, Hq, D), nb, ms * 1e-3),
        tokens_per_s=B / (ms * 1e-3),
        kv_bytes_per_sequence_vs_swa_ring=Skv / 128)
    return res


def bench_backward(args, swa, acc, torch):
    """swa_sink_backward (dq, dk, dv, dsink; bf16) on the 32K SWA prefill
    workload and on a 16K global causal layer, against the forward call."""
    from sliding_window_learnable_amd import inputs
    res = {"workload": "swa_sink_backward bf16, B=1 Hq=64 Hkv=8 D=128: window 128 at S=32768 "
                       "and global causal (window = S) at S=16384",
           "flop_rule": "10 D per attended (row, head, key): q.k and dO.v recomputed, dq, dk, dv"}
    B, Hq, Hkv, D = 1, 64, 8, 128
    for name, S, W, steps in (("swa_32768", 32768, 128, 40), ("global_16384", 16384, 16384, 6)):
        q, k, v, sink = inputs.attention_inputs(2, 0, B, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
        g = inputs.upstream_grad(2, 0, B, S, Hq, D, torch.bfloat16, "cuda")
        out = torch.empty_like(q)
        lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
        if W < S:
            fwd = lambda i: swa.swa_sink_prefill(q, k, v, sink, W, out=out, lse=lse)
        else:
            fwd = lambda i: swa.global_sink_attn(q, k, v, sink, out=out, lse=lse)
        fwd(0)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dsink = torch.empty_like(sink)
        ws = torch.empty(swa.swa_sink_backward_workspace_bytes(B, Hq, S), device="cuda",
                         dtype=torch.uint8)
        log("backward %s: %d steps" % (name, steps))
        ms_b = timed(lambda i: swa.swa_sink_backward(q, k, v, sink, out, lse, g, W, dq=dq, dk=dk,
                                                     dv=dv, dsink=dsink, workspace=ws),
                     steps, max(2, steps // 4))
        ms_f = timed(fwd, steps, max(2, steps // 4))
        fl = acc.backward_flops(B, S, Hq, D, min(W, S))
        nb = acc.backward_bytes(B, S, Hq, Hkv, D)
        res[name] = dict(ms=ms_b, tflops=fl / (ms_b * 1e-3) / 1e12,
                         frac_mfma_peak=fl / (ms_b * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS,
                         frac_roofline=acc.roofline_frac(fl, nb, ms_b * 1e-3),
                         hbm_gbs=nb / (ms_b * 1e-3) / 1e9, forward_ms=ms_f,
                         backward_over_forward=ms_b / ms_f, tokens_per_s=B * S / (ms_b * 1e-3))
        del q, k, v, sink, g, out, lse, dq, dk, dv, dsink, ws
        torch.cuda.empty_cache()
    return res


def bench_varlen(args, swa, acc, torch):
    """swa_sink_prefill_varlen on one context-length bucket: 16 sequences with
    lengths uniform in [512, 8192], packed, as a window-128 layer and as a
    global causal layer; against the same batch padded to the longest length
    and run through the uniform-batch entry points."""
    from sliding_window_learnable_amd import inputs
    Hq, Hkv, D, W = 64, 8, 128, 128
    lengths = [int(n) for n in inputs.cache_lengths(16, 512, 8192, seed=6000)]
    S_max, total = max(lengths), sum(lengths)
    res = {"workload": "packed bf16 batch of 16 sequences, lengths uniform in [512, 8192] "
                       "(seed 6000; %d tokens, longest %d), Hq=64 Hkv=8 D=128" % (total, S_max),
           "lengths": lengths}
    q, k, v, sink, cu = inputs.packed_inputs(6, 0, lengths, Hq, Hkv, D, torch.bfloat16, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty((Hq, total), device="cuda", dtype=torch.float32)
    B = len(lengths)
    for name, win, steps in (("swa_window_128", W, 100), ("global_causal", S_max, 10)):
        log("varlen %s: %d steps" % (name, steps))
        ms = timed(lambda i: swa.swa_sink_prefill_varlen(q, k, v, sink, cu, S_max, win, out=out,
                                                         lse=lse), steps, max(3, steps // 5))
        pairs = sum(acc.window_pairs(n, win) for n in lengths)
        fl = 4 * D * Hq * pairs
        nb = acc.prefill_bytes(1, total, Hq, Hkv, D)
        res[name] = dict(ms=ms, tokens_per_s=total / (ms * 1e-3),
                         tflops=fl / (ms * 1e-3) / 1e12,
                         frac_mfma_peak=fl / (ms * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS,
                         hbm_gbs=nb / (ms * 1e-3) / 1e9,
                         frac_hbm_peak=nb / (ms * 1e-3) / 1e9 / acc.PEAK_HBM_GBS,
                         frac_roofline=acc.roofline_frac(fl, nb, ms * 1e-3))
    del out, lse
    # the same sequences padded on the right to S_max, as a [B, S_max] batch
    qp = torch.zeros((B, S_max, Hq, D), device="cuda", dtype=torch.bfloat16)
    kp = torch.zeros((B, S_max, Hkv, D), device="cuda", dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    offs = [0]
    for n in lengths:
        offs.append(offs[-1] + n)
    for b, n in enumerate(lengths):
        qp[b, :n], kp[b, :n], vp[b, :n] = q[offs[b]:offs[b + 1]], k[offs[b]:offs[b + 1]], \
            v[offs[b]:offs[b + 1]]
    del q, k, v
    outp = torch.empty_like(qp)
    lsep = torch.empty((B, Hq, S_max), device="cuda", dtype=torch.float32)
    log("varlen: padded batch, window 128 and global")
    ms_w = timed(lambda i: swa.swa_sink_prefill(qp, kp, vp, sink, W, out=outp, lse=lsep), 100, 20)
    ms_g = timed(lambda i: swa.global_sink_attn(qp, kp, vp, sink, out=outp, lse=lsep), 10, 3)
    res["swa_window_128"]["padded_batch_ms"] = ms_w
    res["global_causal"]["padded_batch_ms"] = ms_g
    del qp, kp, vp, outp, lsep, sink, cu
    torch.cuda.empty_cache()
    return res


def bench_oracle_configs(args, swa, acc, torch, result):
    """The fp64 oracle beside the GPU on every benchmarked configuration: wall
    time on the host cores, GFLOP/s, the GPU's speed-up (GPU times from the
    sections above) and the largest |GPU - oracle| over the compared outputs.
    Full runs where they take seconds; stated row or sequence samples,
    extrapolated by flops, for the 64K layers, the 256K prefill and the 256K
    global decode.  Config 1 is also timed on one thread."""
    import numpy as np
    import oracle
    from sliding_window_learnable_amd import inputs
    f64 = lambda t: t.double().cpu().numpy()
    nthreads = oracle.threads()
    res = {"threads": nthreads, "affinity_cores": len(os.sched_getaffinity(0)),
           "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}

    def entry(oracle_s, flops, flops_total, gpu_s, err, sample):
        scale = flops_total / flops
        e = {"oracle_s": oracle_s, "oracle_gflops": flops / oracle_s / 1e9, "sample": sample,
             "max_abs_err_vs_gpu": err}
        if scale != 1.0:
            e["oracle_s_extrapolated"] = oracle_s * scale
        if gpu_s is not None:
            e["gpu_s"] = gpu_s
            e["gpu_speedup"] = oracle_s * scale / gpu_s
        return e

    def clock(fn):
        t = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t

    # 1: tiny fp32 reference and its variants; all threads, then one thread
    q, k, v, sink = inputs.attention_inputs(1, 0, 1, 512, 512, 1, 1, 64, torch.float32, "cuda")
    for name, W, sk in (("1", 128, None), ("1_sink=-inf", 128, float("-inf")),
                        ("1_window=512", 512, None)):
        sk_t = sink if sk is None else torch.full_like(sink, sk)
        out, _ = swa.swa_sink_prefill(q, k, v, sk_t, W)
        gpu_ms = timed(lambda i: swa.swa_sink_prefill(q, k, v, sk_t, W), 20, 5)
        args64 = (f64(q), f64(k), f64(v), f64(sk_t), W)
        (ref, _), dt = clock(lambda: oracle.swa_prefill(*args64))
        fl = acc.prefill_flops(1, 512, 1, 64, W)
        res[name] = entry(dt, fl, fl, gpu_ms * 1e-3, float(np.abs(f64(out) - ref).max()), "full")
        if name == "1":
            oracle.set_threads(1)
            _, dt1 = clock(lambda: oracle.swa_prefill(*args64))
            oracle.set_threads(nthreads)
            res[name]["oracle_s_one_thread"] = dt1
    log("oracle beside config 1 done")

    # 3a / 3b: ring decode, full batch of one input set
    for T in (1, 4):
        q, kc, vc, sink = inputs.ring_inputs(3, 0, 256, T, 64, 8, 128, 128, torch.bfloat16, "cuda")
        out, _ = swa.swa_sink_decode(q, kc, vc, sink)
        (ref, _), dt = clock(lambda: oracle.ring_decode(f64(q), f64(kc), f64(vc), f64(sink)))
        fl = acc.decode_flops(256, T, 64, 128, 128)
        gpu = result.get("decode", {}).get("T_q=%d" % T, {}).get("us_per_call")
        res["3_T_q=%d" % T] = entry(dt, fl, fl, None if gpu is None else gpu * 1e-6,
                                    float(np.abs(f64(out) - ref).max()), "full (B=256)")
        del q, kc, vc, sink, out
    log("oracle beside config 3 done")

    # 4: the 64K global layer on every 64th query row, all heads; the SWA
    # layer on 4096 evenly spaced rows
    S, Hq, Hkv, D = 65536, 64, 8, 128
    q, k, v, sink = inputs.attention_inputs(4, 5, 1, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    out, _ = swa.global_sink_attn(q, k, v, sink)
    stride = max(1, int(args.oracle_ga_stride))
    rows = np.arange(0, S, stride)
    idx = torch.as_tensor(rows, device=q.device)
    k64, v64 = f64(k[0][None]), f64(v[0][None])
    (ref, _), dt = clock(lambda: oracle.global_rows(f64(q[0].index_select(0, idx)),
                                                    np.zeros(len(rows)), rows, k64, v64, f64(sink)))
    fl = int(4 * D * Hq * (rows + 1).sum())
    gpu = result.get("hybrid_5to1", {}).get("global_layer_ms")
    res["4_global_layer"] = entry(dt, fl, acc.global_flops(1, S, S, Hq, D),
                                  None if gpu is None else gpu * 1e-3,
                                  float(np.abs(f64(out[0].index_select(0, idx)) - ref).max()),
                                  "every %dth query row (%d rows), all 64 heads; extrapolated by "
                                  "flops" % (stride, len(rows)))
    del q, k, v, sink, out, k64, v64
    q, k, v, sink = inputs.attention_inputs(4, 0, 1, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    out, _ = swa.swa_sink_prefill(q, k, v, sink, 128)
    rows = np.arange(0, S, S // 4096)
    idx = torch.as_tensor(rows, device=q.device)
    (ref, _), dt = clock(lambda: oracle.swa_prefill_rows(
        f64(q[0].index_select(0, idx)), np.zeros(len(rows)), rows, f64(k), f64(v), f64(sink), 128))
    fl = int(4 * D * Hq * np.minimum(rows + 1, 128).sum())
    gpu = result.get("hybrid_5to1", {}).get("swa_layer_ms")
    res["4_swa_layer"] = entry(dt, fl, acc.prefill_flops(1, S, Hq, D, 128),
                               None if gpu is None else gpu * 1e-3,
                               float(np.abs(f64(out[0].index_select(0, idx)) - ref).max()),
                               "4096 evenly spaced query rows, all heads; extrapolated by flops")
    del q, k, v, sink, out
    log("oracle beside config 4 done")

    # 5a: 256K SWA prefill, 4096 rows; 5b: 256K global decode, sequence 0 of 8
    S = 262144
    q, k, v, sink = inputs.attention_inputs(5, 0, 1, S, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    out, _ = swa.swa_sink_prefill(q, k, v, sink, 128)
    rows = np.arange(0, S, S // 4096)
    idx = torch.as_tensor(rows, device=q.device)
    (ref, _), dt = clock(lambda: oracle.swa_prefill_rows(
        f64(q[0].index_select(0, idx)), np.zeros(len(rows)), rows, f64(k), f64(v), f64(sink), 128))
    fl = int(4 * D * Hq * np.minimum(rows + 1, 128).sum())
    gpu = result.get("long_context", {}).get("swa_prefill_262144", {}).get("ms")
    res["5a_swa_prefill_262144"] = entry(dt, fl, acc.prefill_flops(1, S, Hq, D, 128),
                                         None if gpu is None else gpu * 1e-3,
                                         float(np.abs(f64(out[0].index_select(0, idx)) - ref).max()),
                                         "4096 evenly spaced query rows, all heads; extrapolated by flops")
    del q, k, v, sink, out
    q, k, v, sink = inputs.attention_inputs(5, 1, 8, 1, S, Hq, Hkv, D, torch.bfloat16, "cuda")
    out, _ = swa.global_sink_attn(q, k, v, sink)
    k64, v64 = f64(k[0:1]), f64(v[0:1])
    (ref, _), dt = clock(lambda: oracle.global_rows(f64(q[0]), np.zeros(1), np.array([S - 1]),
                                                    k64, v64, f64(sink)))
    fl = acc.global_flops(1, 1, S, Hq, D)
    gpu = result.get("long_context", {}).get("global_decode_B8_262144", {}).get("ms")
    res["5b_global_decode_262144"] = entry(dt, fl, acc.global_flops(8, 1, S, Hq, D),
                                           None if gpu is None else gpu * 1e-3,
                                           float(np.abs(f64(out[0]) - ref).max()),
                                           "sequence 0 of 8, all heads; extrapolated by flops")
    del q, k, v, sink, out, k64, v64
    torch.cuda.empty_cache()
    log("oracle beside config 5 done")
    return res


def bench_copy(args, torch):
    """Plain 1 GiB device copy: the reference kernel for scaling PMC byte counters."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda i: dst.copy_(src), 5, 2)
    return {"bytes_read": n, "bytes_written": n, "ms": ms, "gbs": 2 * n / (ms * 1e-3) / 1e9}


# --------------------------------------------------------------------------- main

def main():
    args = parse_args()
    global SETTLE_S
    SETTLE_S = max(0.0, args.settle_ms) / 1e3
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)." % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import sliding_window_learnable_amd as swa
    from sliding_window_learnable_amd import _lib
    from sliding_window_learnable_amd import accounting as acc
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    _lib.load()                              # fails loudly if the HIP library is missing

    if args.only == "copy":
        print(json.dumps({"copy": bench_copy(args, torch)}))
        return

    result = {}
    if args.only in ("all", "prefill"):
        pre = bench_prefill(args, swa, acc, torch)
        tensors = pre.pop("tensors")
        traffic = traffic_record()
        result.update({
            "metric": METRIC,
            "value": pre["tflops"],
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "clock_settle_ms": args.settle_ms,
            "ms_per_step": pre["ms"],
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16 q/k/v, N(0,1) fp32 sink)",
            "config": {"workload": "swa_sink_prefill B=1 S=32768 Hq=64 Hkv=8 D=128 window=128 "
                                   "bf16 in, fp32 accumulate, bf16 out + fp32 lse",
                       "B": 1, "S": 32768, "Hq": 64, "Hkv": 8, "D": 128, "window": 128},
            "prefill": {k: v for k, v in pre.items() if k != "ms"},
            "roofline": {"bound": "hbm", "achieved": pre["gbs"], "peak": acc.PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": pre["gbs"] / acc.PEAK_HBM_GBS,
                         "traffic": traffic,
                         "kernel": "swa_prefill_ring_kernel<128, 8>",
                         "algorithmic_bytes_per_launch": pre["bytes"]},
        })
        if not args.no_cpu_baseline:
            cb = bench_cpu_baseline(args, acc, torch, tensors)
            cb["gpu_speedup"] = pre["tflops"] / cb["value"]
            result["cpu_baseline"] = cb
        del tensors
        torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        result["decode"] = bench_decode(args, swa, acc, torch)
    if args.only in ("all", "hybrid"):
        result["hybrid_5to1"] = bench_hybrid(args, swa, acc, torch)
    if args.only in ("all", "long"):
        result["long_context"] = bench_long(args, swa, acc, torch)
    if args.only in ("all", "backward"):
        result["backward"] = bench_backward(args, swa, acc, torch)
    if args.only in ("all", "varlen"):
        result["varlen"] = bench_varlen(args, swa, acc, torch)
    if args.only == "all" and not args.no_cpu_baseline:
        result["oracle_by_config"] = bench_oracle_configs(args, swa, acc, torch, result)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
