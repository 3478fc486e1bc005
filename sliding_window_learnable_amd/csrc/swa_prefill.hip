// swa_prefill.hip -- causal sliding-window prefill with a per-head sink,
// bf16 in / fp32 accumulate / bf16 out, for windows up to 129 keys.
//
// Method: "MiMo-V2-Flash Technical Report" digest, 前置知识 / 混合注意力机制
// (each token attends only to a local window, O(n*w) work) and
// 前置知识 / 注意力sink偏置 (a learnable per-head term in every softmax
// denominator); window 128 per 核心方法.  GQA per "小米罗福莉 ... ICML 2026", §02.
//
// Work decomposition (one work-group = one (batch, KV head, chunk of
// positions)):
//  * the G query heads that share a KV head are served by the waves of one
//    work-group, so every K/V byte staged in LDS is used by all G heads;
//  * the chunk is walked in steps of 32 query positions; a step needs the
//    key tiles T1-ntw+1 .. T1 (32 keys each, T1 = the step's own tile), which
//    live in an LDS ring of ntw+1 tiles -- each step loads ONE new tile
//    (prefetched into registers while the current step computes), so K and
//    V cross HBM about once plus a (window-1)-key halo per chunk;
//  * per wave and head: S^T = K Q^T on bf16 MFMA for all ntw tiles at once,
//    band mask, one softmax pass seeded with the sink (running max starts at
//    s_h, denominator at exp(s_h - max)), O^T = V^T P^T on MFMA, then
//    out = O / l (bf16, RNE) and lse = max + ln l.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kTile = 32;
constexpr int kMaxTiles = 5;             // ceil((129-1)/32) + 1
constexpr int kRing = kMaxTiles + 1;     // + the tile being prefetched
constexpr int kRingKeys = kRing * kTile;

template <int D>
struct RingSmem {
    bf16 k[kRing][kTile][D + 8];
    bf16 vt[D][kRingKeys + 8];
};

template <int D, int NT>
struct Stager {
    static constexpr int CH = D / 8;                       // 16-byte chunks per row
    static constexpr int KPT = (kTile * CH + NT - 1) / NT; // K chunks per thread
    static constexpr int VPT = (8 * CH + NT - 1) / NT;     // V quads per thread
    bf16x8 kreg[KPT];
    bf16x8 vreg[VPT][4];

    __device__ __forceinline__ void load(const bf16 *kb, const bf16 *vb, size_t row_stride,
                                         int S, int T, int tid) {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = tid + i * NT;
            kreg[i] = z;
            if (item < kTile * CH) {
                const int pos = kTile * T + item / CH, ch = item % CH;
                if (pos < S) kreg[i] = *(const bf16x8 *)(kb + (size_t)pos * row_stride + 8 * ch);
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int item = tid + i * NT;
#pragma unroll
            for (int j = 0; j < 4; ++j) vreg[i][j] = z;
            if (item < 8 * CH) {
                const int kq = item & 7, ch = item >> 3;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int pos = kTile * T + 4 * kq + j;
                    if (pos < S) vreg[i][j] = *(const bf16x8 *)(vb + (size_t)pos * row_stride + 8 * ch);
                }
            }
        }
    }

    __device__ __forceinline__ void store(RingSmem<D> &sm, int slot, int tid) const {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = tid + i * NT;
            if (item < kTile * CH)
                *(bf16x8 *)&sm.k[slot][item / CH][8 * (item % CH)] = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int item = tid + i * NT;
            if (item < 8 * CH) {
                const int kq = item & 7, ch = item >> 3;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bf16x4 w;
                    w[0] = vreg[i][0][e];
                    w[1] = vreg[i][1][e];
                    w[2] = vreg[i][2][e];
                    w[3] = vreg[i][3][e];
                    *(bf16x4 *)&sm.vt[8 * ch + e][slot * kTile + 4 * kq] = w;
                }
            }
        }
    }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void swa_prefill_ring_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ sink, bf16 *__restrict__ out, float *__restrict__ lse, int S,
    int Hq, int Hkv, int W, int ntw, int chunk) {
    constexpr int NT = NW * 64;
    __shared__ __align__(16) RingSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hl = lane >> 5;
    const int g = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv;
    const int R = ntw + 1;
    const int c0 = blockIdx.x * chunk;
    const int c1 = min(S, c0 + chunk);
    const float c = kLog2e / sqrtf((float)D);

    const size_t row_stride = (size_t)Hkv * D;
    const bf16 *kb = k + ((size_t)b * S * Hkv + g) * D;
    const bf16 *vb = v + ((size_t)b * S * Hkv + g) * D;

    Stager<D, NT> st;
    {
        const int T1 = c0 / kTile;
        for (int T = max(0, T1 - ntw + 1); T <= T1; ++T) {
            st.load(kb, vb, row_stride, S, T, tid);
            st.store(sm, T % R, tid);
        }
    }
    __syncthreads();

    for (int p0 = c0; p0 < c1; p0 += kTile) {
        const int T1 = p0 / kTile;
        const bool has_next = p0 + kTile < c1;
        if (has_next) st.load(kb, vb, row_stride, S, T1 + 1, tid);

        const int pq = p0 + lq;                      // this lane's query position
        const int pqc = min(pq, S - 1);
        for (int hh = wave; hh < G; hh += NW) {
            const int h = g * G + hh;
            const bf16 *qrow = q + (((size_t)b * S + pqc) * Hq + h) * D + 8 * hl;
            bf16x8 qf[D / 16];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 16 * ks);

            // S^T tiles (keys x queries), masked to the band [pq - W + 1, pq].
            f32x16 s[kMaxTiles];
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < kMaxTiles; ++t) {
                const int T = T1 - ntw + 1 + t;
                if (t < ntw && T >= 0) {
                    const int slot = T % R;
                    f32x16 acc = zero16();
                    const bf16 *krow = &sm.k[slot][score_row_key(lq)][8 * hl];
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks)
                        acc = mfma32(*(const bf16x8 *)(krow + 16 * ks), qf[ks], acc);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kp = kTile * T + score_reg_key(r, lane);
                        const bool ok = kp <= pq && kp > pq - W;
                        acc[r] = ok ? acc[r] : -INFINITY;
                        mx = fmaxf(mx, acc[r]);
                    }
                    s[t] = acc;
                }
            }
            mx = wave_xor32_max(mx);

            // Sink-seeded softmax (log2 domain): max starts at s_h, and the
            // denominator carries exp(s_h - max) for the virtual sink token.
            const float s2 = sink[h] * kLog2e;
            const float m = fmaxf(mx * c, s2);
            const float mu = (m == -INFINITY) ? 0.0f : m;
            float l = 0.0f;
#pragma unroll
            for (int t = 0; t < kMaxTiles; ++t) {
                const int T = T1 - ntw + 1 + t;
                if (t < ntw && T >= 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = __builtin_amdgcn_exp2f(fmaf(s[t][r], c, -mu));
                        s[t][r] = p;
                        l += p;
                    }
                }
            }
            l = wave_xor32_sum(l) + __builtin_amdgcn_exp2f(s2 - mu);

            // O^T = V^T P^T.
            f32x16 o[D / 32];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();
#pragma unroll
            for (int t = 0; t < kMaxTiles; ++t) {
                const int T = T1 - ntw + 1 + t;
                if (t < ntw && T >= 0) {
                    const int slot = T % R;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const bf16x8 pb = pack8(s[t], kk);
#pragma unroll
                        for (int dt = 0; dt < D / 32; ++dt) {
                            const bf16x8 a = *(const bf16x8 *)&sm.vt[32 * dt + lq]
                                                                    [slot * kTile + 16 * kk + 8 * hl];
                            o[dt] = mfma32(a, pb, o[dt]);
                        }
                    }
                }
            }

            if (pq < S) {
                const float inv = l > 0.0f ? 1.0f / l : 0.0f;
                bf16 *orow = out + (((size_t)b * S + pq) * Hq + h) * D;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        bf16x4 w;
#pragma unroll
                        for (int e = 0; e < 4; ++e) w[e] = (bf16)(o[dt][4 * j + e] * inv);
                        *(bf16x4 *)(orow + 32 * dt + 8 * j + 4 * hl) = w;
                    }
                }
                if (lse != nullptr && hl == 0)
                    lse[((size_t)b * Hq + h) * S + pq] =
                        l > 0.0f ? (mu + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
            }
        }

        if (has_next) st.store(sm, (T1 + 1) % R, tid);
        __syncthreads();
    }
}

template <int D, int NW>
hipError_t launch_ring(const PrefillArgs &a, hipStream_t stream) {
    const int tiles = (a.S + kTile - 1) / kTile;
    const int groups = a.B * a.Hkv;
    const int target = 256;                                   // one resident work-group per CU
    int per_group = (target + groups - 1) / groups;
    per_group = max(1, min(per_group, tiles));
    int steps = (tiles + per_group - 1) / per_group;
    steps = max(steps, min(4, tiles));
    const int chunk = steps * kTile;
    const int nchunks = (a.S + chunk - 1) / chunk;
    const int ntw = (a.window - 1 + kTile - 1) / kTile + 1;
    dim3 grid(nchunks, a.Hkv, a.B);
    hipLaunchKernelGGL((swa_prefill_ring_kernel<D, NW>), grid, dim3(NW * 64), 0, stream,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.sink,
                       (bf16 *)a.out, a.lse, a.S, a.Hq, a.Hkv, a.window, ntw, chunk);
    return hipGetLastError();
}

template <int D>
hipError_t launch_ring_d(const PrefillArgs &a, hipStream_t stream) {
    switch (waves_for_group(a.Hq / a.Hkv)) {
    case 8: return launch_ring<D, 8>(a, stream);
    case 4: return launch_ring<D, 4>(a, stream);
    case 2: return launch_ring<D, 2>(a, stream);
    default: return launch_ring<D, 1>(a, stream);
    }
}

}  // namespace

bool prefill_ring_supported(int window) { return window >= 1 && window <= 129; }

hipError_t launch_prefill_ring_bf16(const PrefillArgs &a, hipStream_t stream) {
    return a.D == 64 ? launch_ring_d<64>(a, stream) : launch_ring_d<128>(a, stream);
}

}  // namespace swa
