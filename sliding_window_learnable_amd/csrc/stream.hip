// stream.hip -- causal (optionally banded) attention with a per-head sink
// that streams key tiles through LDS: the global full-attention layers
// (technical-report digest, 前置知识 / 混合注意力机制: global layers see the
// whole sequence) and sliding windows too wide for the LDS ring.
//
// One work-group = (batch, KV head, block of 32 query rows); its waves are
// the G query heads of the group, so each K/V tile staged in LDS serves all
// of them.  Queries are aligned to the end of the keys: row i sits at
// position S_kv - S_q + i.  Per 32-key tile and wave:
//   S^T = K Q^T (bf16 MFMA), band/causal mask on boundary tiles only,
//   online softmax whose running max starts at the sink s_h, with lazy
//   rescaling (the accumulator is rescaled only when the running max of
//   some column grows by more than 2^8, so exp2 arguments stay <= 8),
//   O^T += V^T P^T (bf16 MFMA).
// At the end the sink's exp(s_h - max) joins the denominator exactly once.
// Tiles are double-buffered: tile T+1 is fetched into registers while tile
// T is computed.  Work-groups are issued longest-first (the last query
// blocks have the most keys) with the (batch, KV head) index fastest, so
// the blocks of one KV head share an XCD and its L2.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kTile = 32;
constexpr float kRescaleSlack = 8.0f;    // log2 units

template <int D>
struct StreamSmem {
    bf16 k[2][kTile][D + 8];
    bf16 vt[2][D][kTile + 8];
};

template <int D, int NT>
struct TileLoader {
    static constexpr int CH = D / 8;
    static constexpr int KPT = (kTile * CH + NT - 1) / NT;
    static constexpr int VPT = (8 * CH + NT - 1) / NT;
    bf16x8 kreg[KPT];
    bf16x8 vreg[VPT][4];

    __device__ __forceinline__ void load(const bf16 *kb, const bf16 *vb, size_t row_stride,
                                         int S_kv, int T, int tid) {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = tid + i * NT;
            kreg[i] = z;
            if (item < kTile * CH) {
                const int pos = kTile * T + item / CH, ch = item % CH;
                if (pos < S_kv) kreg[i] = *(const bf16x8 *)(kb + (size_t)pos * row_stride + 8 * ch);
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
                    if (pos < S_kv) vreg[i][j] = *(const bf16x8 *)(vb + (size_t)pos * row_stride + 8 * ch);
                }
            }
        }
    }

    __device__ __forceinline__ void store(StreamSmem<D> &sm, int slot, int tid) const {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = tid + i * NT;
            if (item < kTile * CH) *(bf16x8 *)&sm.k[slot][item / CH][8 * (item % CH)] = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int item = tid + i * NT;
            if (item < 8 * CH) {
                const int kq = item & 7, ch = item >> 3;
                u32x2 w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bf16x4 x;
                    x[0] = vreg[i][0][e];
                    x[1] = vreg[i][1][e];
                    x[2] = vreg[i][2][e];
                    x[3] = vreg[i][3][e];
                    w[e] = __builtin_bit_cast(u32x2, x);
                    *(u32x2 *)&sm.vt[slot][8 * ch + e][4 * kq] = w[e];
                }
                // Issued while this step's PV products may still be running.
                lds_settle(w);
            }
        }
    }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void stream_attn_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ sink, bf16 *__restrict__ out, float *__restrict__ lse, int S_q,
    int S_kv, int Hq, int Hkv, int W, int BG, int NB) {
    constexpr int NT = NW * 64;
    __shared__ __align__(16) StreamSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lq = lane & 31, hl = lane >> 5;
    const int bg = blockIdx.x % BG;
    const int qb = NB - 1 - blockIdx.x / BG;          // longest query blocks first
    const int b = bg / Hkv, g = bg % Hkv;
    const int G = Hq / Hkv;
    const float c = kLog2e / sqrtf((float)D);

    const int i0 = qb * kTile;                         // first query row of the block
    const long off = (long)S_kv - S_q;                 // row i sits at position off + i
    const long p_first = off + i0;
    const long p_last = off + min(S_q - 1, i0 + kTile - 1);
    const int T_lo = (int)max(0L, (p_first - W + 1) >= 0 ? (p_first - W + 1) / kTile : 0L);
    const int T_hi = (int)(p_last / kTile);

    const size_t row_stride = (size_t)Hkv * D;
    const bf16 *kb = k + ((size_t)b * S_kv * Hkv + g) * D;
    const bf16 *vb = v + ((size_t)b * S_kv * Hkv + g) * D;

    const int i = i0 + lq;                             // this lane's query row
    const bool row_ok = i < S_q;
    const long pq = off + min(i, S_q - 1);

    TileLoader<D, NT> ld;
    ld.load(kb, vb, row_stride, S_kv, T_lo, tid);
    ld.store(sm, 0, tid);
    lds_barrier();

    for (int hh = wave; hh < G; hh += NW) {
        const int h = g * G + hh;
        bf16x8 qf[D / 16];
        {
            const bf16 *qrow = q + (((size_t)b * S_q + min(i, S_q - 1)) * Hq + h) * D + 8 * hl;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 16 * ks);
        }
        const float s2 = sink[h] * kLog2e;
        float m = s2;                                  // running max seeded with the sink
        float l = 0.0f;                                // this lane's share of the real-token sum
        f32x16 o[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();

        for (int T = T_lo; T <= T_hi; ++T) {
            const int slot = (T - T_lo) & 1;
            const bool prefetch = T < T_hi;
            if (prefetch) ld.load(kb, vb, row_stride, S_kv, T + 1, tid);

            f32x16 s = zero16();
            const bf16 *krow = &sm.k[slot][score_row_key(lq)][8 * hl];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) s = mfma32(*(const bf16x8 *)(krow + 16 * ks), qf[ks], s);

            const long k0 = (long)kTile * T;
            const bool interior = k0 + kTile - 1 <= p_first && k0 >= p_last - W + 1;
            float mx = -INFINITY;
            if (interior) {
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const long kp = k0 + score_reg_key(r, lane);
                    const bool ok = kp <= pq && kp > pq - W;
                    s[r] = ok ? s[r] : -INFINITY;
                    mx = fmaxf(mx, s[r]);
                }
            }
            mx = wave_xor32_max(mx) * c;

            // Lazy rescale: only when some column's max grew by > 2^slack.
            if (__ballot(mx > m + kRescaleSlack) != 0) {
                const float m_new = fmaxf(m, mx);
                const float alpha = (m_new == -INFINITY || m == -INFINITY)
                                        ? (m_new == -INFINITY ? 1.0f : 0.0f)
                                        : __builtin_amdgcn_exp2f(m - m_new);
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
                m = m_new;
            }
            const float mu = (m == -INFINITY) ? 0.0f : m;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -mu));
                s[r] = p;
                l += p;
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 pb = pack8(s, kk);
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const bf16x8 a = *(const bf16x8 *)&sm.vt[slot][32 * dt + lq][16 * kk + 8 * hl];
                    o[dt] = mfma32(a, pb, o[dt]);
                }
            }
            if (prefetch) ld.store(sm, slot ^ 1, tid);
            lds_barrier();
        }

        // Sink joins the denominator once: l_total = sum_j e^{x_j - m} + e^{s_h - m}.
        const float mu = (m == -INFINITY) ? 0.0f : m;
        const float lt = wave_xor32_sum(l) + __builtin_amdgcn_exp2f(s2 - mu);
        if (row_ok) {
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            bf16 *orow = out + (((size_t)b * S_q + i) * Hq + h) * D;
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
                lse[((size_t)b * Hq + h) * S_q + i] =
                    lt > 0.0f ? (mu + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
        }
        if (hh + NW < G) {
            // next head of this wave: restage the first tile
            lds_barrier();
            ld.load(kb, vb, row_stride, S_kv, T_lo, tid);
            ld.store(sm, 0, tid);
            lds_barrier();
        }
    }
}

template <int D, int NW>
hipError_t launch(const PrefillArgs &a, hipStream_t stream) {
    const int BG = a.B * a.Hkv;
    const int NB = (a.S + kTile - 1) / kTile;
    const long n_wg = (long)BG * NB;
    hipLaunchKernelGGL((stream_attn_kernel<D, NW>), dim3((unsigned)n_wg), dim3(NW * 64), 0, stream,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.sink,
                       (bf16 *)a.out, a.lse, a.S, a.S_kv, a.Hq, a.Hkv, a.window, BG, NB);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t stream) {
    switch (waves_for_group(a.Hq / a.Hkv)) {
    case 8: return launch<D, 8>(a, stream);
    case 4: return launch<D, 4>(a, stream);
    case 2: return launch<D, 2>(a, stream);
    default: return launch<D, 1>(a, stream);
    }
}

}  // namespace

hipError_t launch_stream_bf16(const PrefillArgs &a, hipStream_t stream) {
    return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace swa
