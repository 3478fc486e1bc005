// launch.h -- internal (C++) interface between the C ABI entry points and
// the kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

struct PrefillArgs {            // also used for global attention
    const void *q, *k, *v;
    const float *sink;
    void *out;
    float *lse;
    int B, Hq, Hkv;
    int S;                      // query rows per sequence (S_q)
    int S_kv;                   // key rows per sequence
    int D;
    int window;                 // keys per row, counting the row itself
    const int32_t *cu_seqlens = nullptr;   // packed varlen batch: [B+1] row offsets (S = max length)
    int total = 0;              // rows of the packed batch
};

struct DecodeArgs {
    const void *q, *kcache, *vcache;
    const float *sink;
    void *out;
    float *lse;
    const int32_t *cache_len;   // may be NULL: L = R (every ring full)
    int B, Hq, Hkv, T, W, D;    // W: keys per query (window)
    int R;                      // ring slots (>= W)
};

// RoPE on the T new queries and keys at positions L_old + t, keys and
// values written to ring slots (L_old + t) mod R.
struct AppendArgs {
    const void *q, *k_new, *v_new;
    void *q_rot, *kcache, *vcache;
    const int32_t *cache_len_old;   // may be NULL: L_old = 0
    int B, Hq, Hkv, T, R, D;
    double theta;
};
hipError_t launch_rope_append(const AppendArgs &a, bool bf16, hipStream_t stream);

// bf16 sliding-window prefill, LDS ring of key tiles (98 <= window <= 129).
bool prefill_ring_supported(int window, int G);
int prefill_chunk_cap(int Hq, int Hkv, int D, int ntw);
hipError_t launch_prefill_ring_bf16(const PrefillArgs &a, hipStream_t stream);

// bf16 banded / causal attention streaming key tiles through LDS: any window,
// queries aligned to the end of the keys (row i at position S_kv - S + i).
hipError_t launch_stream_bf16(const PrefillArgs &a, hipStream_t stream);
// The same, also writing per (query head, 32-row block, block_k-key block)
// the largest scaled logit over the block's visible pairs to bmax
// [B, Hq, ceil(S/32), ceil(S_kv/block_k)] (block_k a multiple of 32).
hipError_t launch_stream_bf16_block_max(const PrefillArgs &a, float *bmax, int block_k,
                                        hipStream_t stream);

// bf16 decode over a ring cache (split-free).
hipError_t launch_ring_decode_bf16(const DecodeArgs &a, hipStream_t stream);

// bf16 split-KV partials over a linear cache + combine (sink added once).
struct SplitPlan {
    int n_splits;               // key ranges per (sequence, KV head, column tile)
    int kps;                    // keys per range (a multiple of 32)
    int n_ct;                   // 32-column tiles of (token, head) pairs
};
SplitPlan plan_split(int B, int Hq, int Hkv, int S_q, int S_kv, int D);
int splitkv_num_splits(int B, int Hq, int Hkv, int S_q, int S_kv);
bool splitkv_preferred(int Hq, int Hkv, int S_q, int S_kv);
size_t splitkv_workspace_bytes(int B, int Hq, int Hkv, int S_q, int S_kv, int D);
hipError_t launch_splitkv_bf16(const PrefillArgs &a, void *workspace, hipStream_t stream);
// The same with the partials in the library's static per-device scratch
// array (kStaticScratchBytes); the caller checks the size first.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t launch_splitkv_bf16_static(const PrefillArgs &a, hipStream_t stream);

// Backward of causal sliding-window / global attention with a sink.
struct BackwardArgs {
    const void *q, *k, *v;
    const float *sink;
    const void *out;            // forward output
    const float *lse;           // forward lse [B, Hq, S]
    const void *dout;
    void *dq, *dk, *dv;
    float *dsink;
    float *ws_dsum;             // [B, Hq, S]: D_i = dO_i . O_i
    float *ws_l2;               // [B, Hq, S]: lse_i * log2(e)
    float *ws_part;             // [B, Hq, ceil(S/32)]: sink-gradient partials
    int B, Hq, Hkv, S, D, window;
};
constexpr int kBackwardRows = 32;      // rows per sink-gradient partial
size_t backward_workspace_bytes(int B, int Hq, int S);
hipError_t launch_backward_pre(const BackwardArgs &a, hipStream_t stream, bool bf16_inputs);
// dsink_h = -(sum of the per-32-row partials in ws_part), fixed order.
hipError_t launch_backward_dsink(const BackwardArgs &a, hipStream_t stream);
hipError_t launch_backward_f32(const BackwardArgs &a, hipStream_t stream);
hipError_t launch_backward_bf16(const BackwardArgs &a, hipStream_t stream);

// float32 path (one wavefront per query row and head), every call type.
hipError_t launch_generic_f32_linear(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_generic_f32_ring(const DecodeArgs &a, hipStream_t stream);

}  // namespace swa
