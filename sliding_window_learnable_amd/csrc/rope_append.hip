// rope_append.hip -- the step before ring decode: rotary position embedding
// of the T_q new queries and keys at their absolute positions, and the keys
// (rotated) and values written to their ring slots.
//
// Sources: "小米罗福莉：MiMo-V2.5如何做到又快又强又便宜？| ICML 2026", Q&A on
// RoPE (positions keep increasing as the window slides, so cached keys carry
// absolute positions); the technical-report digest, 前置知识 / 多token预测
// (1 + 3 draft tokens per step, verified in one pass).  With a ring of at
// least window + T_q - 1 slots, rejected drafts are rolled back by the caller
// lowering its token count: the slots they took are rewritten by the next
// step, and no position a later query needs was overwritten.
//
// Rotation (the pages name RoPE but not its layout): dimension i pairs with
// i + D/2 at angle P * theta^(-2i/D); the angle is formed and reduced modulo
// 2 pi in double precision (P reaches 2^20 and beyond), then applied in
// fp32 to every query and key head.
#include <cmath>

#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

// One work-group per (sequence, token): the D/2 angles are formed once
// (double precision, reduced modulo 2 pi) into LDS, then the work-group's
// threads rotate 8-dim chunks of every query head and key head and copy the
// value rows, with 8-element vector loads and stores.
template <class T>
__global__ __launch_bounds__(256) void rope_append_kernel(
    const T *__restrict__ q, const T *__restrict__ k_new, const T *__restrict__ v_new,
    T *q_rot, T *__restrict__ kc, T *__restrict__ vc, const int32_t *__restrict__ cache_len_old,
    int Hq, int Hkv, int Tq, int R, int D, double theta) {
    typedef T V8 __attribute__((ext_vector_type(8)));
    __shared__ float cs[64], sn[64];
    const int tid = threadIdx.x;
    const int t = blockIdx.x % Tq, b = blockIdx.x / Tq;
    const int half = D / 2, CH = half / 8;                 // 8-dim chunks per half
    const long P = (cache_len_old ? (long)cache_len_old[b] : 0L) + t;
    if (tid < half) {
        const double two_pi = 6.283185307179586476925286766559;
        double a = (double)P * pow(theta, -2.0 * (double)tid / (double)D);
        a -= floor(a / two_pi) * two_pi;
        cs[tid] = (float)cos(a);
        sn[tid] = (float)sin(a);
    }
    __syncthreads();
    // Non-negative for any P, so a malformed (negative) cache_len_old still
    // lands inside this sequence's ring.
    const int slot = (int)(((P % R) + R) % R);
    const int nq = Hq * CH, nk = Hkv * CH, nv = Hkv * 2 * CH;
    for (int it = tid; it < nq + nk + nv; it += blockDim.x) {
        if (it < nq + nk) {
            const bool is_q = it < nq;
            const int hh = is_q ? it / CH : (it - nq) / CH, c = (is_q ? it : it - nq) % CH;
            const T *src = is_q ? q + (((size_t)b * Tq + t) * Hq + hh) * D
                                : k_new + (((size_t)b * Tq + t) * Hkv + hh) * D;
            T *dst = is_q ? q_rot + (((size_t)b * Tq + t) * Hq + hh) * D
                          : kc + (((size_t)b * Hkv + hh) * R + slot) * D;
            const V8 x0 = *(const V8 *)(src + 8 * c), x1 = *(const V8 *)(src + half + 8 * c);
            V8 y0, y1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a0 = (float)x0[e], a1 = (float)x1[e];
                const float co = cs[8 * c + e], si = sn[8 * c + e];
                y0[e] = (T)(a0 * co - a1 * si);
                y1[e] = (T)(a1 * co + a0 * si);
            }
            *(V8 *)(dst + 8 * c) = y0;                     // q_rot may be q: read above
            *(V8 *)(dst + half + 8 * c) = y1;
        } else {
            const int j = it - nq - nk, g = j / (2 * CH), c = j % (2 * CH);
            *(V8 *)(vc + (((size_t)b * Hkv + g) * R + slot) * D + 8 * c) =
                *(const V8 *)(v_new + (((size_t)b * Tq + t) * Hkv + g) * D + 8 * c);
        }
    }
}

template <class T>
hipError_t launch_t(const AppendArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(rope_append_kernel<T>, dim3((unsigned)(a.B * a.T)), dim3(256), 0, stream,
                       (const T *)a.q, (const T *)a.k_new, (const T *)a.v_new, (T *)a.q_rot,
                       (T *)a.kcache, (T *)a.vcache, a.cache_len_old, a.Hq, a.Hkv, a.T, a.R, a.D,
                       a.theta);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_append(const AppendArgs &a, bool bf16_data, hipStream_t stream) {
    return bf16_data ? launch_t<bf16>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace swa
