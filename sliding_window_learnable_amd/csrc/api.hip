// api.hip -- the extern "C" entry points declared in include/swa_sink.h:
// argument validation (before any HIP call), dispatch to the kernel
// launchers, and status codes.
#include "swa_sink.h"

#include <cmath>

#include "launch.h"

namespace {

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool dtype_ok(int dtype) { return dtype == SWA_F32 || dtype == SWA_BF16; }

bool head_dim_ok(int D) { return D == 64 || D == 128; }

// Grid dimensions y and z carry heads and batch.
constexpr int kMaxGridYZ = 65535;

int common_checks(int B, int Hq, int Hkv, int D, int dtype) {
    if (B < 0 || Hq < 1 || Hkv < 1 || D < 1) return SWA_ERR_SHAPE;
    if (Hq % Hkv != 0) return SWA_ERR_SHAPE;
    if (B > kMaxGridYZ || Hq > kMaxGridYZ) return SWA_ERR_SHAPE;
    if (!dtype_ok(dtype) || !head_dim_ok(D)) return SWA_ERR_UNSUPPORTED;
    return SWA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? SWA_OK : SWA_ERR_HIP; }

// Work-groups / work items of one launch must fit a 31-bit grid dimension.
constexpr long kMaxGridX = 0x7fffffffL;
bool grid_fits(long units) { return units >= 0 && units <= kMaxGridX; }

// Row counts (sequence lengths, packed totals, query tokens) are at most
// 2^30, so that position arithmetic in the kernels (a position plus a tile
// or a window) stays inside 32-bit integers.
constexpr int kMaxRows = 1 << 30;
bool rows_ok(long n) { return n >= 0 && n <= kMaxRows; }

// 32-row blocks of n rows, without overflow.
long blocks32(int n) { return ((long)n + 31) / 32; }

}  // namespace

extern "C" {

int swa_sink_prefill(const void *q, const void *k, const void *v, const float *sink, void *out,
                     float *lse, int B, int Hq, int Hkv, int S, int D, int window, int dtype,
                     void *stream) {
    if (!q || !k || !v || !sink || !out) return SWA_ERR_NULL;
    if (!rows_ok(S) || window < 1) return SWA_ERR_SHAPE;
    const int rc = common_checks(B, Hq, Hkv, D, dtype);
    if (rc != SWA_OK) return rc;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(sink, 4) || !aligned(lse, 4))
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || S == 0) return SWA_OK;
    if (!grid_fits((long)B * Hkv * blocks32(S) * (Hq / Hkv))) return SWA_ERR_SHAPE;
    if (window > S) window = S;                       // every key of the sequence: same result

    swa::PrefillArgs a{q, k, v, sink, out, lse, B, Hq, Hkv, S, S, D, window};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == SWA_F32) return status_of(swa::launch_generic_f32_linear(a, st));
    if (swa::prefill_ring_supported(window, Hq / Hkv)) return status_of(swa::launch_prefill_ring_bf16(a, st));
    return status_of(swa::launch_stream_bf16(a, st));
}

int swa_sink_prefill_varlen(const void *q, const void *k, const void *v, const float *sink,
                            void *out, float *lse, const int32_t *cu_seqlens, int B,
                            int max_seqlen, int total, int Hq, int Hkv, int D, int window,
                            int dtype, void *stream) {
    if (!q || !k || !v || !sink || !out || !cu_seqlens) return SWA_ERR_NULL;
    if (!rows_ok(max_seqlen) || !rows_ok(total) || window < 1) return SWA_ERR_SHAPE;
    const int rc = common_checks(B, Hq, Hkv, D, dtype);
    if (rc != SWA_OK) return rc;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(sink, 4) || !aligned(lse, 4) || !aligned(cu_seqlens, 4))
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || max_seqlen == 0 || total == 0) return SWA_OK;
    if (!grid_fits((long)B * Hkv * blocks32(max_seqlen) * (Hq / Hkv))) return SWA_ERR_SHAPE;
    if (window > max_seqlen) window = max_seqlen;     // every key of each sequence

    swa::PrefillArgs a{q, k, v, sink, out, lse, B, Hq, Hkv, max_seqlen, max_seqlen, D,
                       window, cu_seqlens, total};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == SWA_F32) return status_of(swa::launch_generic_f32_linear(a, st));
    if (swa::prefill_ring_supported(window, Hq / Hkv))
        return status_of(swa::launch_prefill_ring_bf16(a, st));
    return status_of(swa::launch_stream_bf16(a, st));
}

int swa_sink_decode(const void *q, const void *kcache, const void *vcache, const float *sink,
                    void *out, float *lse, int B, int Hq, int Hkv, int T_q, int window, int D,
                    const int32_t *cache_len, int dtype, void *stream) {
    if (!q || !kcache || !vcache || !sink || !out) return SWA_ERR_NULL;
    if (!rows_ok(T_q) || window < 1 || T_q > window) return SWA_ERR_SHAPE;
    const int rc = common_checks(B, Hq, Hkv, D, dtype);
    if (rc != SWA_OK) return rc;
    if (!aligned(q, 16) || !aligned(kcache, 16) || !aligned(vcache, 16) || !aligned(out, 16) ||
        !aligned(sink, 4) || !aligned(lse, 4) || !aligned(cache_len, 4))
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || T_q == 0) return SWA_OK;
    if (!grid_fits((long)B * Hq * T_q)) return SWA_ERR_SHAPE;
    if ((long)window * D * 2 > kMaxGridX) return SWA_ERR_UNSUPPORTED;   // one ring's buffer window

    swa::DecodeArgs a{q, kcache, vcache, sink, out, lse, cache_len, B, Hq, Hkv, T_q, window, D,
                      window};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == SWA_F32) return status_of(swa::launch_generic_f32_ring(a, st));
    return status_of(swa::launch_ring_decode_bf16(a, st));
}

int swa_sink_decode_ring(const void *q, const void *kcache, const void *vcache, const float *sink,
                         void *out, float *lse, int B, int Hq, int Hkv, int T_q, int window,
                         int ring, int D, const int32_t *cache_len, int dtype, void *stream) {
    if (!q || !kcache || !vcache || !sink || !out) return SWA_ERR_NULL;
    if (!rows_ok(T_q) || window < 1 || ring < window || T_q > ring) return SWA_ERR_SHAPE;
    const int rc = common_checks(B, Hq, Hkv, D, dtype);
    if (rc != SWA_OK) return rc;
    if (!aligned(q, 16) || !aligned(kcache, 16) || !aligned(vcache, 16) || !aligned(out, 16) ||
        !aligned(sink, 4) || !aligned(lse, 4) || !aligned(cache_len, 4))
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || T_q == 0) return SWA_OK;
    if (!grid_fits((long)B * Hq * T_q)) return SWA_ERR_SHAPE;
    if ((long)ring * D * 2 > kMaxGridX) return SWA_ERR_UNSUPPORTED;     // one ring's buffer window

    swa::DecodeArgs a{q, kcache, vcache, sink, out, lse, cache_len, B, Hq, Hkv, T_q, window, D,
                      ring};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == SWA_F32) return status_of(swa::launch_generic_f32_ring(a, st));
    return status_of(swa::launch_ring_decode_bf16(a, st));
}

int swa_sink_rope_append(const void *q, const void *k_new, const void *v_new, void *q_rot,
                         void *kcache, void *vcache, const int32_t *cache_len_old, int B, int Hq,
                         int Hkv, int T_q, int ring, int D, double rope_theta, int dtype,
                         void *stream) {
    if (!q || !k_new || !v_new || !q_rot || !kcache || !vcache) return SWA_ERR_NULL;
    if (!rows_ok(T_q) || ring < 1 || T_q > ring) return SWA_ERR_SHAPE;
    const int rc = common_checks(B, Hq, Hkv, D, dtype);
    if (rc != SWA_OK) return rc;
    if (!(rope_theta > 1.0) || !std::isfinite(rope_theta)) return SWA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(q_rot, 16) ||
        !aligned(kcache, 16) || !aligned(vcache, 16) || !aligned(cache_len_old, 4))
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || T_q == 0) return SWA_OK;
    if (!grid_fits((long)B * T_q)) return SWA_ERR_SHAPE;

    swa::AppendArgs a{q, k_new, v_new, q_rot, kcache, vcache, cache_len_old,
                      B, Hq, Hkv, T_q, ring, D, rope_theta};
    return status_of(swa::launch_rope_append(a, dtype == SWA_BF16, static_cast<hipStream_t>(stream)));
}

size_t global_sink_attn_workspace_bytes(int B, int Hq, int Hkv, int S_q, int S_kv, int D) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S_q < 1 || S_kv < S_q ||
        !rows_ok(S_kv) || !head_dim_ok(D))
        return 0;
    if (!swa::splitkv_preferred(Hq, Hkv, S_q, S_kv)) return 0;
    return swa::splitkv_workspace_bytes(B, Hq, Hkv, S_q, S_kv, D);
}

int global_sink_attn(const void *q, const void *k, const void *v, const float *sink, void *out,
                     float *lse, int B, int Hq, int Hkv, int S_q, int S_kv, int D,
                     void *workspace, size_t workspace_bytes, int dtype, void *stream) {
    if (!q || !k || !v || !sink || !out) return SWA_ERR_NULL;
    if (!rows_ok(S_q) || !rows_ok(S_kv) || S_q > S_kv) return SWA_ERR_SHAPE;
    const int rc = common_checks(B, Hq, Hkv, D, dtype);
    if (rc != SWA_OK) return rc;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(sink, 4) || !aligned(lse, 4))
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || S_q == 0) return SWA_OK;
    if (!grid_fits((long)B * Hkv * blocks32(S_q) * (Hq / Hkv))) return SWA_ERR_SHAPE;

    // Every key position is inside the window: window = S_kv.
    swa::PrefillArgs a{q, k, v, sink, out, lse, B, Hq, Hkv, S_q, S_kv, D, S_kv};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == SWA_F32) return status_of(swa::launch_generic_f32_linear(a, st));
    if (swa::splitkv_preferred(Hq, Hkv, S_q, S_kv)) {
        const size_t need = swa::splitkv_workspace_bytes(B, Hq, Hkv, S_q, S_kv, D);
        if (workspace == nullptr || workspace_bytes < need) return SWA_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return SWA_ERR_UNSUPPORTED;
        return status_of(swa::launch_splitkv_bf16(a, workspace, st));
    }
    return status_of(swa::launch_stream_bf16(a, st));
}

int global_sink_attn_noalloc(const void *q, const void *k, const void *v, const float *sink,
                             void *out, float *lse, int B, int Hq, int Hkv, int S_q, int S_kv,
                             int D, int dtype, void *stream) {
    if (!q || !k || !v || !sink || !out) return SWA_ERR_NULL;
    if (!rows_ok(S_q) || !rows_ok(S_kv) || S_q > S_kv) return SWA_ERR_SHAPE;
    const int rc = common_checks(B, Hq, Hkv, D, dtype);
    if (rc != SWA_OK) return rc;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(sink, 4) || !aligned(lse, 4))
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || S_q == 0) return SWA_OK;
    if (!grid_fits((long)B * Hkv * blocks32(S_q) * (Hq / Hkv))) return SWA_ERR_SHAPE;

    swa::PrefillArgs a{q, k, v, sink, out, lse, B, Hq, Hkv, S_q, S_kv, D, S_kv};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == SWA_F32) return status_of(swa::launch_generic_f32_linear(a, st));
    if (swa::splitkv_preferred(Hq, Hkv, S_q, S_kv)) {
        if (swa::splitkv_workspace_bytes(B, Hq, Hkv, S_q, S_kv, D) > swa::kStaticScratchBytes)
            return SWA_ERR_SCRATCH;
        return status_of(swa::launch_splitkv_bf16_static(a, st));
    }
    return status_of(swa::launch_stream_bf16(a, st));
}

int global_sink_attn_block_max(const void *q, const void *k, const void *v, const float *sink,
                               void *out, float *lse, float *block_max, int block_k, int B,
                               int Hq, int Hkv, int S_q, int S_kv, int D, int dtype,
                               void *stream) {
    if (!q || !k || !v || !sink || !out || !block_max) return SWA_ERR_NULL;
    if (!rows_ok(S_q) || !rows_ok(S_kv) || S_q > S_kv || block_k < 32 || block_k % 32 != 0)
        return SWA_ERR_SHAPE;
    const int rc = common_checks(B, Hq, Hkv, D, dtype);
    if (rc != SWA_OK) return rc;
    if (dtype != SWA_BF16) return SWA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(sink, 4) || !aligned(lse, 4) || !aligned(block_max, 4))
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || S_q == 0) return SWA_OK;
    if (!grid_fits((long)B * Hkv * blocks32(S_q) * (Hq / Hkv))) return SWA_ERR_SHAPE;

    swa::PrefillArgs a{q, k, v, sink, out, lse, B, Hq, Hkv, S_q, S_kv, D, S_kv};
    return status_of(
        swa::launch_stream_bf16_block_max(a, block_max, block_k, static_cast<hipStream_t>(stream)));
}

size_t swa_sink_backward_workspace_bytes(int B, int Hq, int S) {
    if (B < 1 || Hq < 1 || S < 1 || !rows_ok(S)) return 0;
    return swa::backward_workspace_bytes(B, Hq, S);
}

int swa_sink_backward(const void *q, const void *k, const void *v, const float *sink,
                      const void *out, const float *lse, const void *dout, void *dq, void *dk,
                      void *dv, float *dsink, int B, int Hq, int Hkv, int S, int D, int window,
                      void *workspace, size_t workspace_bytes, int dtype, void *stream) {
    if (!q || !k || !v || !sink || !out || !lse || !dout || !dq || !dk || !dv || !dsink)
        return SWA_ERR_NULL;
    if (!rows_ok(S) || window < 1) return SWA_ERR_SHAPE;
    const int rc = common_checks(B, Hq, Hkv, D, dtype);
    if (rc != SWA_OK) return rc;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(sink, 4) || !aligned(lse, 4) || !aligned(dsink, 4))
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || S == 0) return SWA_OK;
    if (!grid_fits((long)B * Hq * S)) return SWA_ERR_SHAPE;
    const size_t need = swa::backward_workspace_bytes(B, Hq, S);
    if (workspace == nullptr || workspace_bytes < need) return SWA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return SWA_ERR_UNSUPPORTED;

    float *ws = static_cast<float *>(workspace);
    const size_t rows = (size_t)B * Hq * S;
    swa::BackwardArgs a{q,  k,  v,  sink, out, lse, dout, dq, dk, dv, dsink, ws, ws + rows,
                        ws + 2 * rows, B, Hq, Hkv, S, D, window < S ? window : S};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == SWA_F32) return status_of(swa::launch_backward_f32(a, st));
    return status_of(swa::launch_backward_bf16(a, st));
}

const char *swa_sink_strerror(int code) {
    switch (code) {
    case SWA_OK: return "success";
    case SWA_ERR_NULL: return "a required pointer argument is NULL";
    case SWA_ERR_SHAPE:
        return "invalid sizes (negative size, more than 2^30 rows, Hq % Hkv != 0, window < 1, "
               "T_q > window, S_q > S_kv, batch/heads above 65535, or more work units than one "
               "launch holds)";
    case SWA_ERR_UNSUPPORTED:
        return "unsupported argument (head dim not 64/128, unknown dtype, a pointer not "
               "aligned to 16 bytes, or a ring cache above 2 GiB per (sequence, KV head))";
    case SWA_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case SWA_ERR_HIP: return "the HIP runtime reported an error when launching";
    case SWA_ERR_SCRATCH:
        return "the sizes need more scratch than the static 64 MiB array of "
               "global_sink_attn_noalloc holds";
    default: return "unknown status code";
    }
}

}  // extern "C"
