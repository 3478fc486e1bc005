// attn_device.h -- device building blocks shared by the gfx950 attention
// kernels: bf16 MFMA tiles, operand layouts, LDS staging and the
// sink-seeded softmax state.
//
// MFMA tile used everywhere: v_mfma_f32_32x32x16_bf16 (64-lane wavefront).
//   A (32 x 16): lane l holds row (l & 31), k-elements 8*(l >> 5) + e, e = 0..7
//   B (16 x 32): lane l holds col (l & 31), k-elements 8*(l >> 5) + e
//   C (32 x 32): lane l holds col (l & 31), rows 8*(r >> 2) + 4*(l >> 5) + (r & 3)
//                for accumulator register r = 0..15.
// Scores are computed transposed, S^T = K Q^T (rows = keys, cols = queries),
// so that every lane owns one query column: row reductions become in-lane
// reductions plus one exchange with lane l ^ 32, and the score registers are
// already laid out as the B operand of the next product O^T = V^T P^T.
// To make that hand-off free, the A rows of S^T are fed keys in the order
//   row m = 8j + 4h + c  <-  key 16*(j >> 1) + 8*h + 4*(j & 1) + c
// after which accumulator register r of lane l holds the key
//   16*(r >> 3) + 8*(l >> 5) + (r & 7)
// i.e. registers 0..7 are 8 consecutive keys = one B operand of a K=16 step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// Key index (0..31 within a 32-key tile) that A row m of S^T is fed with.
__device__ __forceinline__ int score_row_key(int m) {
    const int j = m >> 3, h = (m >> 2) & 1, c = m & 3;
    return 16 * (j >> 1) + 8 * h + 4 * (j & 1) + c;
}

// Key index (0..31) held by accumulator register r of lane `lane` in S^T.
__device__ __forceinline__ int score_reg_key(int r, int lane) {
    return 16 * (r >> 3) + 8 * (lane >> 5) + (r & 7);
}

// Row (0..31 within a 32-row d-tile) of output register r of lane `lane`.
__device__ __forceinline__ int out_reg_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16 &p, int half) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (bf16)p[8 * half + e];
    return b;
}

__device__ __forceinline__ float wave_xor32_max(float x) {
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_xor32_sum(float x) {
    return x + __shfl_xor(x, 32);
}

// Largest power of two dividing G, capped at 8: waves per work-group when
// one wave serves one query head of a GQA group.
__host__ __device__ constexpr int waves_for_group(int G) {
    return (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

// ---------------------------------------------------------------------------
// LDS staging of a 32-key tile.
//
// K tile : [32 keys][D + 8] bf16 (16-byte row pad: the 8 rows that one
//          ds_read_b128 quarter-wave touches land on distinct bank groups).
// V^T    : [D][ring keys + 8] bf16, keys contiguous, so one 16-byte read
//          gives the 8 consecutive keys of an A operand of O^T = V^T P^T.
// ---------------------------------------------------------------------------

// Global -> register prefetch of one K chunk (16 bytes) per thread item.
template <int D>
struct KChunk {
    bf16x8 val;
    int key, chunk;
    bool live;
};

// V^T staging item: 4 keys x 8 dims (four 16-byte rows), written to LDS as
// eight 8-byte stores, one per dim, each holding 4 consecutive keys.
struct VQuad {
    bf16x8 rows[4];
    int kq, chunk;
    bool live;
};

}  // namespace swa
