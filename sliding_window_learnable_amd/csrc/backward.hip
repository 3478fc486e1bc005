// backward.hip -- gradients of causal sliding-window / global attention with
// a learnable per-head sink: dq, dk, dv and dsink for an upstream gradient dO.
//
// The sink s_h is a learned per-head term in every softmax denominator
// (technical-report digest, 前置知识 / 注意力sink偏置); its gradient follows
// from a virtual key with logit s_h and a zero value vector:
//   P_ij = e^{x_ij - lse_i},  p_sink,i = e^{s_h - lse_i}  (lse from the forward)
//   dv_j += P_ij dO_i,        dP_ij = dO_i . v_j,   D_i = dO_i . O_i
//   dx_ij = P_ij (dP_ij - D_i),   ds_h = -sum_i p_sink,i D_i
//   dq_i = scale sum_j dx_ij k_j,   dk_j = scale sum_i dx_ij q_i
//
// Passes: (1) bwd_pre: D_i and per-32-row partials of the sink gradient;
// (2) dsink: the partials of each head summed in a fixed order
// (deterministic, no atomics); (3) dq and (4) dk/dv, each owning its
// outputs, so no pass accumulates into another's memory.  This file holds
// passes 1-2 and the float32 path of 3-4 (one wave per output row); the
// bf16 MFMA kernels of 3-4 are in backward_mfma.hip.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kRows = kBackwardRows;     // rows per pre-pass work unit

// Dot product of one 16-byte piece of two rows (8 bf16 or 4 float elements).
__device__ __forceinline__ float dot16(const bf16 *x, const bf16 *y) {
    const bf16x8 a = *(const bf16x8 *)x, c = *(const bf16x8 *)y;
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)a[e] * (float)c[e];
    return s;
}
__device__ __forceinline__ float dot16(const float *x, const float *y) {
    const f32x4 a = *(const f32x4 *)x, c = *(const f32x4 *)y;
    return a[0] * c[0] + a[1] * c[1] + a[2] * c[2] + a[3] * c[3];
}

// One wave per (32 rows, head, batch): D_i = dO_i . O_i for each row, and the
// sum over those rows of e^{s_h - lse_i} D_i.  Each row is read as one
// contiguous segment: LPR lanes x 16 bytes, 64/LPR rows per pass.
template <class T>
__global__ __launch_bounds__(64) void bwd_pre_kernel(const T *__restrict__ out,
                                                     const T *__restrict__ dout,
                                                     const float *__restrict__ lse,
                                                     const float *__restrict__ sink,
                                                     float *__restrict__ dsum, float *__restrict__ l2,
                                                     float *__restrict__ part, int S, int Hq, int D) {
    constexpr int EPC = 16 / sizeof(T);              // elements per 16-byte piece
    const int LPR = D / EPC;                         // lanes per row (8..32)
    const int RPP = 64 / LPR;                        // rows per pass
    const int lane = threadIdx.x, sub = lane % LPR, rsel = lane / LPR;
    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const float s = sink[h];
    float term = 0.0f;                               // valid in lanes with sub == 0
    for (int r0 = 0; r0 < kRows; r0 += RPP) {
        const int i = tile * kRows + r0 + rsel;
        const bool ok = i < S;
        float acc = 0.0f;
        if (ok) {
            const size_t row = (((size_t)b * S + i) * Hq + h) * D + (size_t)sub * EPC;
            acc = dot16(out + row, dout + row);
        }
        for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m);
        if (ok && sub == 0) {
            const size_t li = ((size_t)b * Hq + h) * S + i;
            dsum[li] = acc;
            l2[li] = lse[li] * kLog2e;
            if (s != -INFINITY) term += expf(s - lse[li]) * acc;
        }
    }
    term = sub == 0 ? term : 0.0f;
    for (int m = 1; m < 64; m <<= 1) term += __shfl_xor(term, m);
    if (lane == 0) part[((size_t)b * Hq + h) * gridDim.x + tile] = term;
}

// dsink[h] = -(sum over batch and row tiles of the partials), fixed order.
__global__ __launch_bounds__(64) void dsink_kernel(const float *__restrict__ part,
                                                   float *__restrict__ dsink, int B, int Hq,
                                                   int tiles) {
    const int h = blockIdx.x, lane = threadIdx.x;
    float acc = 0.0f;
    for (int b = 0; b < B; ++b)
        for (int t = lane; t < tiles; t += 64) acc += part[((size_t)b * Hq + h) * tiles + t];
    for (int m = 1; m < 64; m <<= 1) acc += __shfl_xor(acc, m);
    if (lane == 0) dsink[h] = -acc;
}

// ---------------------------------------------------------------------------
// float32 path: one wave per output row, keys (or queries) one at a time.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_sum64(float x) {
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

template <class T>
__device__ __forceinline__ float el(const T *p, size_t i, int lane_d, int D) {
    return lane_d < D ? (float)p[i + lane_d] : 0.0f;
}

// dq_i for one (row i, head h, batch b); lane holds dims lane, lane+64.
template <class T>
__global__ __launch_bounds__(64) void gen_dq_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                    const T *__restrict__ v,
                                                    const T *__restrict__ dout,
                                                    const float *__restrict__ lse,
                                                    const float *__restrict__ dsum,
                                                    T *__restrict__ dq, int S, int Hq, int Hkv,
                                                    int D, int W) {
    const int lane = threadIdx.x;
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (Hq / Hkv);
    const float scale = 1.0f / sqrtf((float)D);
    const size_t qrow = (((size_t)b * S + i) * Hq + h) * D;
    const float l = lse[((size_t)b * Hq + h) * S + i];
    const float Di = dsum[((size_t)b * Hq + h) * S + i];
    const float q0 = el(q, qrow, lane, D), q1 = el(q, qrow, lane + 64, D);
    const float g0 = el(dout, qrow, lane, D), g1 = el(dout, qrow, lane + 64, D);
    float a0 = 0.0f, a1 = 0.0f;
    for (int j = max(0, i - W + 1); j <= i; ++j) {
        const size_t krow = (((size_t)b * S + j) * Hkv + g) * D;
        const float k0 = el(k, krow, lane, D), k1 = el(k, krow, lane + 64, D);
        const float v0 = el(v, krow, lane, D), v1 = el(v, krow, lane + 64, D);
        const float x = wave_sum64(q0 * k0 + q1 * k1) * scale;
        const float dp = wave_sum64(g0 * v0 + g1 * v1);
        const float P = expf(x - l);
        const float dx = P * (dp - Di);
        a0 += dx * k0;
        a1 += dx * k1;
    }
    if (lane < D) dq[qrow + lane] = (T)(a0 * scale);
    if (lane + 64 < D) dq[qrow + lane + 64] = (T)(a1 * scale);
}

// dk_j, dv_j for one (key j, KV head g, batch b): every query head of the
// group and every query that sees key j.
template <class T>
__global__ __launch_bounds__(64) void gen_dkdv_kernel(const T *__restrict__ q,
                                                      const T *__restrict__ k,
                                                      const T *__restrict__ v,
                                                      const T *__restrict__ dout,
                                                      const float *__restrict__ lse,
                                                      const float *__restrict__ dsum,
                                                      T *__restrict__ dk, T *__restrict__ dv, int S,
                                                      int Hq, int Hkv, int D, int W) {
    const int lane = threadIdx.x;
    const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv;
    const float scale = 1.0f / sqrtf((float)D);
    const size_t krow = (((size_t)b * S + j) * Hkv + g) * D;
    const float k0 = el(k, krow, lane, D), k1 = el(k, krow, lane + 64, D);
    const float v0 = el(v, krow, lane, D), v1 = el(v, krow, lane + 64, D);
    float ak0 = 0.0f, ak1 = 0.0f, av0 = 0.0f, av1 = 0.0f;
    const int i_end = (int)min((long)S - 1, (long)j + W - 1);
    for (int h = g * G; h < (g + 1) * G; ++h) {
        for (int i = j; i <= i_end; ++i) {
            const size_t qrow = (((size_t)b * S + i) * Hq + h) * D;
            const float q0 = el(q, qrow, lane, D), q1 = el(q, qrow, lane + 64, D);
            const float g0 = el(dout, qrow, lane, D), g1 = el(dout, qrow, lane + 64, D);
            const float l = lse[((size_t)b * Hq + h) * S + i];
            const float Di = dsum[((size_t)b * Hq + h) * S + i];
            const float x = wave_sum64(q0 * k0 + q1 * k1) * scale;
            const float dp = wave_sum64(g0 * v0 + g1 * v1);
            const float P = expf(x - l);
            const float dx = P * (dp - Di);
            av0 += P * g0;
            av1 += P * g1;
            ak0 += dx * q0;
            ak1 += dx * q1;
        }
    }
    if (lane < D) {
        dk[krow + lane] = (T)(ak0 * scale);
        dv[krow + lane] = (T)av0;
    }
    if (lane + 64 < D) {
        dk[krow + lane + 64] = (T)(ak1 * scale);
        dv[krow + lane + 64] = (T)av1;
    }
}

template <class T>
hipError_t launch_pre(const BackwardArgs &a, hipStream_t stream) {
    const int tiles = (a.S + kRows - 1) / kRows;
    hipLaunchKernelGGL(bwd_pre_kernel<T>, dim3(tiles, a.Hq, a.B), dim3(64), 0, stream,
                       (const T *)a.out, (const T *)a.dout, a.lse, a.sink, a.ws_dsum, a.ws_l2,
                       a.ws_part, a.S, a.Hq, a.D);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dsink_kernel, dim3(a.Hq), dim3(64), 0, stream, a.ws_part, a.dsink, a.B,
                       a.Hq, tiles);
    return hipGetLastError();
}

template <class T>
hipError_t launch_generic(const BackwardArgs &a, hipStream_t stream);

}  // namespace

namespace {

template <class T>
hipError_t launch_generic(const BackwardArgs &a, hipStream_t stream) {
    hipError_t e = launch_pre<T>(a, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gen_dq_kernel<T>, dim3(a.S, a.Hq, a.B), dim3(64), 0, stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, (const T *)a.dout, a.lse,
                       a.ws_dsum, (T *)a.dq, a.S, a.Hq, a.Hkv, a.D, a.window);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gen_dkdv_kernel<T>, dim3(a.S, a.Hkv, a.B), dim3(64), 0, stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, (const T *)a.dout, a.lse,
                       a.ws_dsum, (T *)a.dk, (T *)a.dv, a.S, a.Hq, a.Hkv, a.D, a.window);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_f32(const BackwardArgs &a, hipStream_t stream) {
    return launch_generic<float>(a, stream);
}

hipError_t launch_backward_pre(const BackwardArgs &a, hipStream_t stream, bool bf16_inputs) {
    return bf16_inputs ? launch_pre<bf16>(a, stream) : launch_pre<float>(a, stream);
}

hipError_t launch_backward_dsink(const BackwardArgs &a, hipStream_t stream) {
    const int tiles = (a.S + kRows - 1) / kRows;
    hipLaunchKernelGGL(dsink_kernel, dim3(a.Hq), dim3(64), 0, stream, a.ws_part, a.dsink, a.B,
                       a.Hq, tiles);
    return hipGetLastError();
}

}  // namespace swa
