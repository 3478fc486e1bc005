/*
 * swa_sink.h -- C ABI of the MI355X (gfx950) sliding-window + sink attention
 * library (libswa_sink.so).
 *
 * The method (page title, section):
 *  - "MiMo-V2-Flash Technical Report" digest, 前置知识 / 注意力sink偏置
 *    (attention-sink bias): each attention head owns a learnable scalar s_h
 *    that enters the softmax denominator, so attention mass can go to a
 *    virtual sink token instead of real tokens.  The virtual token carries
 *    no value vector.
 *  - same digest, 前置知识 / 混合注意力机制 (hybrid attention) and 核心方法
 *    (core method): sliding-window layers (window 128) interleaved with
 *    global full-attention layers at SWA:GA = 5:1.
 *  - "小米罗福莉：MiMo-V2.5如何做到又快又强又便宜？| ICML 2026", §02 of the
 *    talk: grouped-query attention (GQA) throughout; 7:1 for the larger model.
 *  - pwwt.cn article on MiMo-V2-Flash, §1.1 Hybrid Attention: the
 *    sliding-window KV cache has a fixed size, O(W) memory.
 *
 * For query row i of head h (KV head g = h / (Hq/Hkv)) with key set K_i:
 *     x_j = (1/sqrt(D)) q_i . k_j                   (j in K_i)
 *     out_i = sum_j e^{x_j} v_j / (e^{s_h} + sum_j e^{x_j})
 *     lse_i = ln(e^{s_h} + sum_j e^{x_j})           (natural log, sink included)
 * s_h = -inf gives ordinary softmax attention.  An empty key set gives
 * out = 0, lse = s_h.
 *
 * Conventions shared by every call:
 *  - q, k, v, out and the caches are DEVICE pointers, contiguous, row-major,
 *    all of element type `dtype` (SWA_F32 or SWA_BF16).  `sink` [Hq] and
 *    `lse` are always float32 device pointers.  `cache_len` is an int32
 *    device pointer.
 *  - The caller owns and allocates every buffer; the library never
 *    allocates, frees or synchronises, keeps no mutable global state and is
 *    re-entrant (except global_sink_attn_noalloc, which uses the library's
 *    own static scratch array: see there).  Work is enqueued on `stream`
 *    (a hipStream_t; NULL = the default stream) and results are valid once
 *    the caller synchronises it.
 *  - Every argument is validated before any HIP call; a non-zero return
 *    means nothing was launched (SWA_ERR_HIP: the launch itself failed).
 *    Batch and row counts (B, S, T_q, S_q) may be 0: nothing is launched
 *    and SWA_OK is returned.
 *  - Tensor pointers (q, k, v, out, caches, workspace) must be 16-byte
 *    aligned; sink, lse and cache_len 4-byte aligned (SWA_ERR_UNSUPPORTED).
 *  - GQA: Hq % Hkv == 0; query head h reads KV head h / (Hq/Hkv).
 *  - Softmax scale is fixed at 1/sqrt(D).
 *  - Sink values must be finite or -inf (+inf is undefined).
 *  - Non-finite inputs are not clamped: a NaN sink makes every output of its
 *    head NaN (lse too; a row with no visible key keeps out = 0), a NaN in
 *    a query row makes that row's out and lse NaN, a NaN in a key row makes
 *    out and lse NaN for exactly the rows that see that key.  A non-finite
 *    value row makes out NaN for the rows that see it and may also reach
 *    rows of the same 32-key tile that do not (their weight for it is 0,
 *    and 0 * NaN = NaN in the matrix products); lse is unaffected.
 *  - Supported head dims: D in {64, 128}.
 *  - A window larger than the sequence is the same as the whole sequence.
 *  - bfloat16 results are rounded to nearest-even from float32 accumulators.
 */
#ifndef SWA_SINK_H
#define SWA_SINK_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SWA_API __attribute__((visibility("default")))
#else
#define SWA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum swa_dtype { SWA_F32 = 0, SWA_BF16 = 1 };

enum swa_status {
    SWA_OK = 0,
    SWA_ERR_NULL = -1,        /* a required pointer is NULL                        */
    SWA_ERR_SHAPE = -2,       /* negative size, Hq/Hkv/D/window < 1, Hq % Hkv != 0,
                                 T_q > window, S_q > S_kv, B or Hq > 65535, a row
                                 count (S, S_q, S_kv, T_q, max_seqlen, total) above
                                 2^30, or more work units (B*Hq*rows/32, B*Hq*T_q)
                                 than 2^31-1                                        */
    SWA_ERR_UNSUPPORTED = -3, /* D not in {64,128}, unknown dtype, misaligned pointer,
                                 or window*D*2 > 2^31-1 bytes for one decode ring  */
    SWA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required        */
    SWA_ERR_HIP = -5,         /* the HIP runtime reported an error at launch       */
    SWA_ERR_SCRATCH = -6      /* global_sink_attn_noalloc: the sizes need more than
                                 its static scratch array holds (64 MiB)           */
};

/*
 * Causal sliding-window prefill with a per-head sink.
 * Source: technical-report digest, 前置知识 / 混合注意力机制 and
 * 注意力sink偏置; window 128 per 核心方法.
 *
 *   q    [B, S, Hq, D]    k, v [B, S, Hkv, D]    sink [Hq] (float32)
 *   out  [B, S, Hq, D]    lse  [B, Hq, S] (float32, natural log; may be NULL)
 * Row i sees key positions max(0, i - window + 1) .. i (window keys,
 * including itself).  window >= S gives full causal attention.
 */
SWA_API int swa_sink_prefill(const void *q, const void *k, const void *v, const float *sink,
                     void *out, float *lse, int B, int Hq, int Hkv, int S, int D,
                     int window, int dtype, void *stream);

/*
 * swa_sink_prefill over a packed batch of sequences of different lengths
 * (context-length buckets served together).  Source: "小米罗福莉：MiMo-V2.5
 * 如何做到又快又强又便宜？| ICML 2026", §06 Q&A (audience E: requests are
 * grouped into buckets by context length); the attention itself is that of
 * swa_sink_prefill, applied to each sequence on its own.
 *
 *   q, out  [total, Hq, D]    k, v [total, Hkv, D]    sink [Hq] (float32)
 *   lse     [Hq, total] (float32, natural log; may be NULL)
 *   cu_seqlens  int32 [B + 1] on the device: sequence b is rows
 *               cu_seqlens[b] .. cu_seqlens[b+1] - 1; cu_seqlens[0] = 0,
 *               non-decreasing, cu_seqlens[B] = total, every length
 *               <= max_seqlen.  The kernels clamp each entry to that range,
 *               so a malformed table gives wrong rows but no access outside
 *               the tensors.
 * Row i of a sequence sees its own rows max(0, i - window + 1) .. i; window
 * >= max_seqlen gives causal global attention per sequence.  Zero-length
 * sequences are allowed.  Work-groups for rows past a sequence's end exit at
 * once, so the cost follows max_seqlen * B for the launch and the real rows
 * for the arithmetic.
 */
SWA_API int swa_sink_prefill_varlen(const void *q, const void *k, const void *v,
                                    const float *sink, void *out, float *lse,
                                    const int32_t *cu_seqlens, int B, int max_seqlen,
                                    int total, int Hq, int Hkv, int D, int window,
                                    int dtype, void *stream);

/*
 * Decode over a fixed ring KV cache of `window` slots per (sequence, KV head),
 * with T_q >= 1 new query tokens per sequence (T_q > 1 verifies MTP draft
 * tokens in one pass).  Sources: pwwt.cn article, §1.1 Hybrid Attention
 * (fixed-size SWA KV cache); technical-report digest, 前置知识 / 多token预测
 * (the main model verifies 3 draft tokens in parallel); "小米罗福莉 ...
 * ICML 2026", Q&A on RoPE (positions keep increasing as the window slides).
 *
 *   q       [B, T_q, Hq, D]
 *   kcache  [B, Hkv, window, D]   the key of absolute position P is in slot P % window
 *   vcache  [B, Hkv, window, D]
 *   out     [B, T_q, Hq, D]       lse [B, Hq, T_q] (float32; may be NULL)
 *   cache_len  int32 [B] on the device: L_b = tokens written so far,
 *              INCLUDING the T_q new ones (already written to their slots);
 *              NULL means every ring is exactly full (L = window).
 * Query t is at position p = L - T_q + t and sees positions max(0, L-window)
 * .. p (older positions were overwritten).  With a full ring, draft t sees
 * window - (T_q - 1 - t) keys.  Rows with p < 0 see no key (out = 0).
 * Requires T_q <= window.  The kernel never reads a slot outside the ring,
 * and while the ring is not yet full (L < window) it never reads the slots
 * L .. window-1 that no token has reached, whatever they hold.
 */
SWA_API int swa_sink_decode(const void *q, const void *kcache, const void *vcache,
                    const float *sink, void *out, float *lse, int B, int Hq, int Hkv,
                    int T_q, int window, int D, const int32_t *cache_len, int dtype,
                    void *stream);

/*
 * Ring decode with the attention window separate from the ring size, for
 * MTP draft verification with rollback.  Source: technical-report digest,
 * 前置知识 / 多token预测 (1 + 3 draft tokens verified in one pass) and the
 * pwwt.cn article on MiMo-V2-Flash, §1.1 (fixed-size SWA cache).
 *
 *   kcache, vcache [B, Hkv, ring, D]: position P in slot P mod ring
 *   cache_len [B] (device, int32; NULL: L = ring): tokens written so far,
 *                 including the T_q new ones
 * Query t sits at position p = L - T_q + t and sees positions
 * max(0, L - ring, p - window + 1) .. p.  With ring >= window + T_q - 1
 * every query sees its full window however many drafts the previous step
 * rejected (the caller rolls back by lowering its token count; the rejected
 * slots are rewritten by the next append).  ring == window is exactly
 * swa_sink_decode.  Requires window >= 1, ring >= window, T_q <= ring.
 * Before the ring fills (L < ring) the slots L .. ring-1 are never read.
 * Other arguments and results as for swa_sink_decode.
 */
SWA_API int swa_sink_decode_ring(const void *q, const void *kcache, const void *vcache,
                                 const float *sink, void *out, float *lse, int B, int Hq,
                                 int Hkv, int T_q, int window, int ring, int D,
                                 const int32_t *cache_len, int dtype, void *stream);

/*
 * The step before ring decode: rotary position embedding of the T_q new
 * queries and keys at their absolute positions, and the rotated keys and the
 * values written to their ring slots.  Source: "小米罗福莉：MiMo-V2.5如何做到
 * 又快又强又便宜？| ICML 2026", Q&A on RoPE (positions keep increasing as the
 * window slides: cached keys carry absolute positions).
 *
 *   q, q_rot [B, T_q, Hq, D]   k_new, v_new [B, T_q, Hkv, D]   (dtype)
 *   kcache, vcache [B, Hkv, ring, D]
 *   cache_len_old [B] (device, int32; NULL: 0): tokens in the cache before
 *                 this step; token t is at position P = cache_len_old + t
 *                 (a negative entry is not an error the kernel can report:
 *                 its slots are taken as P mod ring in [0, ring), so the
 *                 writes stay inside that sequence's ring)
 * Rotation: dimension i (< D/2) pairs with i + D/2 at angle
 * P * rope_theta^(-2i/D):  y_i = x_i cos - x_{i+D/2} sin,
 * y_{i+D/2} = x_{i+D/2} cos + x_i sin (angles reduced in double precision,
 * applied in fp32, rounded to dtype).  q_rot may be q (in place); the keys
 * and values of token t go to slot P mod ring.  Requires T_q <= ring and
 * rope_theta > 1 (else SWA_ERR_SHAPE / SWA_ERR_UNSUPPORTED).  The caller
 * then decodes with cache_len_old + T_q tokens.
 */
SWA_API int swa_sink_rope_append(const void *q, const void *k_new, const void *v_new,
                                 void *q_rot, void *kcache, void *vcache,
                                 const int32_t *cache_len_old, int B, int Hq, int Hkv, int T_q,
                                 int ring, int D, double rope_theta, int dtype, void *stream);

/*
 * Workspace (bytes) that global_sink_attn needs for these sizes; 0 means it
 * needs none (the workspace pointer may then be NULL).  The value does not
 * depend on dtype.
 */
SWA_API size_t global_sink_attn_workspace_bytes(int B, int Hq, int Hkv, int S_q, int S_kv, int D);

/*
 * Global (full) causal attention with a per-head sink: the global layers of
 * the hybrid stack.  Source: technical-report digest, 前置知识 / 混合注意力机制
 * (global layers see the whole sequence) and 注意力sink偏置.
 *
 *   q   [B, S_q, Hq, D]     k, v [B, S_kv, Hkv, D]    sink [Hq]
 *   out [B, S_q, Hq, D]     lse  [B, Hq, S_q] (float32; may be NULL)
 * Queries are aligned to the END of the keys: row i sits at position
 * S_kv - S_q + i and sees keys 0 .. that position (S_q == S_kv is prefill,
 * S_q << S_kv is decode).  Short query blocks are split over the keys; the
 * partial results go to `workspace` (device memory of at least
 * global_sink_attn_workspace_bytes(...) bytes) and a combine pass adds the
 * sink exactly once.
 */
SWA_API int global_sink_attn(const void *q, const void *k, const void *v, const float *sink,
                     void *out, float *lse, int B, int Hq, int Hkv, int S_q, int S_kv,
                     int D, void *workspace, size_t workspace_bytes, int dtype,
                     void *stream);

/*
 * global_sink_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and results, with no workspace argument.
 * Where global_sink_attn would use a workspace (short query blocks split over
 * the keys), the partial results go to a static device array of the library
 * instead, 64 MiB per GPU, held from the first such call on that GPU until
 * the process ends.  Sizes whose
 * global_sink_attn_workspace_bytes(...) exceeds 64 MiB return
 * SWA_ERR_SCRATCH before anything is launched.  The call itself allocates
 * nothing (no hipMalloc, no library allocation); its first call on a device
 * looks up that device's copy of the array.  Calls that overlap on one GPU
 * (several streams or threads) share the array and race: serialise them.
 * Each call's partials are written before they are read, so successive calls
 * need no clearing.
 */
SWA_API int global_sink_attn_noalloc(const void *q, const void *k, const void *v,
                                     const float *sink, void *out, float *lse, int B, int Hq,
                                     int Hkv, int S_q, int S_kv, int D, int dtype, void *stream);

/*
 * global_sink_attn plus a block-score side output: for every query head h,
 * 32-row query block qb and key block kb of block_k keys,
 *   block_max[b, h, qb, kb] = max over the visible (row i, key j) of the
 *                             block of q_i . k_j / sqrt(D)   (-inf if none),
 * the scaled logit in the units of the sink s_h, as the full-attention pass
 * forms it tile by tile.  Source: "小米罗福莉：MiMo-V2.5如何做到又快又强又
 * 便宜？| ICML 2026", §02 (High Sparse: sparse layers select tokens by
 * block from the block-level scores of the full-attention layer's
 * FlashAttention pass, at no extra cost).
 *
 *   block_max  float32 [B, Hq, ceil(S_q / 32), ceil(S_kv / block_k)],
 *              every element written (the caller need not clear it)
 *   block_k    key block size: a positive multiple of 32 (else SWA_ERR_SHAPE)
 * Other arguments, layouts and results as for global_sink_attn (queries at
 * the end of the keys); out and lse are bit-identical to it.  bf16 only
 * (SWA_ERR_UNSUPPORTED for float32); no workspace (the prefill-shaped
 * streaming kernel serves every S_q).
 */
SWA_API int global_sink_attn_block_max(const void *q, const void *k, const void *v,
                                       const float *sink, void *out, float *lse,
                                       float *block_max, int block_k, int B, int Hq, int Hkv,
                                       int S_q, int S_kv, int D, int dtype, void *stream);

/*
 * Gradients of swa_sink_prefill (window < S) or of causal global attention
 * with a sink (window >= S, S_q == S_kv == S) for an upstream gradient dout:
 * dq, dk, dv and the gradient of the learnable sink.
 * Source: technical-report digest, 前置知识 / 注意力sink偏置 (the sink is a
 * learnable per-head term of every softmax denominator, i.e. a virtual key
 * with logit s_h and no value); window and causality as for the forward.
 *
 *   q, out, dout, dq [B, S, Hq, D]    k, v, dk, dv [B, S, Hkv, D]
 *   sink, dsink [Hq] (float32)        lse [B, Hq, S] (float32)
 *
 * `out` and `lse` are the forward's outputs for the same inputs.  With
 * P_ij = e^{x_ij - lse_i} and D_i = dout_i . out_i:
 *   dv_j = sum_i P_ij dout_i,   dx_ij = P_ij (dout_i . v_j - D_i),
 *   dq_i = sum_j dx_ij k_j / sqrt(D),   dk_j = sum_i dx_ij q_i / sqrt(D),
 *   dsink_h = -sum_{b,i} e^{s_h - lse_i} D_i     (summed over the batch).
 * dk/dv sum over the query heads of a KV head.  dq, dk, dv (dtype) and dsink
 * are overwritten, not accumulated.  The bf16 path computes in float32 from
 * bf16 operands and rounds the gradients to bf16 (RNE).
 *
 * `workspace`: device memory of at least
 * swa_sink_backward_workspace_bytes(B, Hq, S) bytes, 16-byte aligned
 * (SWA_ERR_WORKSPACE if missing or too small); its contents are scratch.
 * The result is deterministic: no atomics, fixed reduction order.
 */
SWA_API size_t swa_sink_backward_workspace_bytes(int B, int Hq, int S);
SWA_API int swa_sink_backward(const void *q, const void *k, const void *v, const float *sink,
                              const void *out, const float *lse, const void *dout, void *dq,
                              void *dk, void *dv, float *dsink, int B, int Hq, int Hkv, int S,
                              int D, int window, void *workspace, size_t workspace_bytes,
                              int dtype, void *stream);

/* Static, human-readable text for a status code (never NULL). */
SWA_API const char *swa_sink_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SWA_SINK_H */
