// generic_f32.hip -- float32 path for every call type (prefill, global,
// ring decode): one 64-lane wavefront per (query row, head), fp32 throughout.
//
// Method: "MiMo-V2-Flash Technical Report" digest, 前置知识 / 注意力sink偏置
// (learnable per-head term in the softmax denominator) and 混合注意力机制
// (local window / global layers).
//
// Each lane walks keys lo+lane, lo+lane+64, ... with its own running
// (max, denominator, accumulator[D]); the 64 partial states are then merged
// through LDS and the sink enters the merged denominator exactly once.
// This path exists for float32 inputs, where exact fp32 products are wanted;
// the bfloat16 path is the MFMA kernels.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

template <int D, bool RING>
__global__ __launch_bounds__(64) void generic_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ sink, float *__restrict__ out, float *__restrict__ lse,
    int Hq, int Hkv, int rows, int nkeys, int window, const int32_t *__restrict__ cache_len,
    const int32_t *__restrict__ cu, int total) {
    __shared__ float qs[D];
    __shared__ float red[64][D + 1];
    __shared__ float wts[64];

    const int lane = threadIdx.x;
    const int row = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (Hq / Hkv);
    const float c = kLog2e / sqrtf((float)D);

    // Packed variable-length batch (linear mode, cu != nullptr): sequence b
    // is rows cu[b] .. cu[b+1]-1 of [total, H, D]; lse is [Hq, total].
    size_t q_row0 = (size_t)b * rows, kv_row0 = (size_t)b * nkeys;
    if (!RING && cu != nullptr) {
        const int s0 = min(max(cu[b], 0), total);   // clamped against a malformed table
        const int s1 = min(max(cu[b + 1], s0), min(total, s0 + rows));
        rows = nkeys = s1 - s0;
        q_row0 = kv_row0 = (size_t)s0;
        if (row >= rows) return;                       // whole work-group, before any barrier
    }
    const size_t qoff = ((q_row0 + row) * Hq + h) * D;
    for (int d = lane; d < D; d += 64) qs[d] = q[qoff + d];
    __syncthreads();

    long lo, hi;
    if (RING) {   // nkeys = ring slots; positions max(0, L-nkeys, p-window+1) .. p = L-T+row
        const long L = cache_len ? (long)cache_len[b] : (long)nkeys;
        hi = L - rows + row;
        lo = L - nkeys > 0 ? L - nkeys : 0;
        lo = hi - window + 1 > lo ? hi - window + 1 : lo;
    } else {      // rows aligned to the end of the keys
        hi = (long)nkeys - rows + row;
        lo = hi - window + 1 > 0 ? hi - window + 1 : 0;
    }

    float m = -INFINITY, l = 0.0f;
    float acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.0f;
    for (long j = lo + lane; j <= hi; j += 64) {
        size_t off;
        if (RING)
            off = (((size_t)b * Hkv + g) * nkeys + (size_t)(j % nkeys)) * D;
        else
            off = ((kv_row0 + j) * Hkv + g) * D;
        const float *kr = k + off;
        const float *vr = v + off;
        float x = 0.0f;
#pragma unroll 16
        for (int d = 0; d < D; ++d) x = fmaf(qs[d], kr[d], x);
        x *= c;
        if (x > m) {
            const float a = exp2f(m - x);
            l *= a;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] *= a;
            m = x;
        }
        const float p = exp2f(x - m);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vr[d], acc[d]);
    }

    // Merge the 64 lane states; the sink is one more term of the denominator.
    const float s2 = sink[h] * kLog2e;
    float M = m;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    M = fmaxf(M, s2);
    const float Mu = (M == -INFINITY) ? 0.0f : M;
    const float f = exp2f(m - Mu);
    float Lreal = l * f;                               // real-token mass
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) Lreal += __shfl_xor(Lreal, off);
    const float Ltot = Lreal + exp2f(s2 - Mu);
#pragma unroll
    for (int d = 0; d < D; ++d) red[lane][d] = acc[d] * f;
    wts[lane] = 0.0f;
    __syncthreads();
    // No real-token mass leaves out = 0; every other denominator divides (a
    // NaN one included, so non-finite inputs propagate).
    const float inv = Lreal == 0.0f ? 0.0f : 1.0f / Ltot;
    for (int d = lane; d < D; d += 64) {
        float s = 0.0f;
        for (int i = 0; i < 64; ++i) s += red[i][d];
        out[qoff + d] = s * inv;
    }
    if (lse != nullptr && lane == 0)
        lse[(!RING && cu != nullptr ? (size_t)h * total + q_row0 : ((size_t)b * Hq + h) * rows) + row] =
            Ltot == 0.0f ? -INFINITY : (Mu + log2f(Ltot)) * kLn2;
}

template <int D>
hipError_t linear_d(const PrefillArgs &a, hipStream_t stream) {
    dim3 grid(a.S, a.Hq, a.B);
    hipLaunchKernelGGL((generic_f32_kernel<D, false>), grid, dim3(64), 0, stream,
                       (const float *)a.q, (const float *)a.k, (const float *)a.v, a.sink,
                       (float *)a.out, a.lse, a.Hq, a.Hkv, a.S, a.S_kv, a.window,
                       (const int32_t *)nullptr, a.cu_seqlens, a.total);
    return hipGetLastError();
}

template <int D>
hipError_t ring_d(const DecodeArgs &a, hipStream_t stream) {
    dim3 grid(a.T, a.Hq, a.B);
    hipLaunchKernelGGL((generic_f32_kernel<D, true>), grid, dim3(64), 0, stream,
                       (const float *)a.q, (const float *)a.kcache, (const float *)a.vcache,
                       a.sink, (float *)a.out, a.lse, a.Hq, a.Hkv, a.T, a.R, a.W, a.cache_len,
                       (const int32_t *)nullptr, 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_generic_f32_linear(const PrefillArgs &a, hipStream_t stream) {
    return a.D == 64 ? linear_d<64>(a, stream) : linear_d<128>(a, stream);
}

hipError_t launch_generic_f32_ring(const DecodeArgs &a, hipStream_t stream) {
    return a.D == 64 ? ring_d<64>(a, stream) : ring_d<128>(a, stream);
}

}  // namespace swa
