// decode.hip -- short query blocks against a key cache, bf16 MFMA.
//
//  * ring decode: T_q new tokens per sequence against the fixed W-slot
//    sliding-window cache, no split (pwwt.cn article on MiMo-V2-Flash, §1.1
//    Hybrid Attention: the SWA KV cache is fixed-size; technical-report
//    digest, 前置知识 / 多token预测: draft tokens are verified by the main
//    model in one pass).
//  * split-KV partials for global attention over a long linear cache: each
//    wave reduces one key range to an unnormalised (max, sum, acc) without
//    the sink, and a combine pass merges the splits and adds the sink
//    exactly once (technical-report digest, 前置知识 / 注意力sink偏置).
//
// Columns of the MFMA tiles are (token t, head in group) pairs: G*T_q of
// them per (sequence, KV head), 32 per column tile, so the K/V bytes of a
// (sequence, KV head) are read from HBM once for all its heads and draft
// tokens.  Decode is bound by HBM: every wave streams its own keys with the
// next chunk's loads in flight while the current chunk computes, and waves
// never wait on each other, so each CU keeps ~16 KiB per wave in flight.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kChunk = 32;          // keys per step (one S^T tile)
constexpr int kVtPad = 4;           // V^T row padding: conflict-free transposed writes
constexpr int kKtPad = 8;           // K row padding: conflict-free fragment reads
constexpr int kWavesPerWG = 4;      // independent waves per work-group

// Mode RING: keys are ring slots 0..W-1 of [B, Hkv, W, D]; with base =
// (L-1) mod W the slot j holds position L-1-base+j, minus W when j > base,
// visible to token t when it lies in [max(0, L-W, p-Wnd+1), p], p = L-T+t
// (Wnd: the attention window, at most the W slots).  Mode LINEAR:
// keys are positions [k_begin, k_end) of [B, S_kv, Hkv, D] (one split),
// visible to token t when <= S_kv-T+t.
//
// One wave = one work item (column tile ct, split, KV head g, sequence b):
// it streams the item's keys in 32-key chunks, the next chunk's K
// fragments and V rows being loaded into registers while the current chunk
// computes.  Per chunk: S^T = K Q^T (K fragments straight from HBM into the
// A operand), mask, online softmax (running max seeded with the sink in
// RING mode, raised lazily), V^T staged through this wave's own LDS tile,
// O^T += V^T P^T.  Waves never synchronise with each other.
template <int D, bool RING>
__global__ __launch_bounds__(64 * kWavesPerWG, 2) void decode_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ kc, const bf16 *__restrict__ vc,
    const float *__restrict__ sink, bf16 *__restrict__ out, float *__restrict__ lse,
    const int32_t *__restrict__ cache_len, int B, int Hq, int Hkv, int T, int W, int S_kv,
    int kps, int n_ct, int n_splits, float *__restrict__ part, int Wnd) {
    constexpr int KF = D / 16;                     // Q fragments, K loads per lane
    constexpr int VPT = D / 64;                    // V items (4 keys x 8 dims) per lane
    constexpr float kSlack = 8.0f;                 // log2 units
    __shared__ __align__(16) bf16 kt_all[kWavesPerWG][kChunk][D + kKtPad];
    __shared__ __align__(16) bf16 vt_all[kWavesPerWG][D][kChunk + kVtPad];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lq = lane & 31, hl = lane >> 5;
    const int item = blockIdx.x * kWavesPerWG + wave;
    if (item >= n_ct * n_splits * Hkv * B) return;          // wave-uniform
    const int ct = item % n_ct;
    const int split = (item / n_ct) % n_splits;
    const int g = (item / (n_ct * n_splits)) % Hkv;
    const int b = item / (n_ct * n_splits * Hkv);
    const int G = Hq / Hkv;
    bf16 (*kt)[D + kKtPad] = kt_all[wave];
    bf16 (*vt)[kChunk + kVtPad] = vt_all[wave];
    const float c = kLog2e / sqrtf((float)D);

    // This lane's column: token t, query head h.
    const int n = 32 * ct + lq;
    const bool col_ok = n < G * T;
    const int nc = col_ok ? n : 0;
    const int t = nc / G, h = g * G + nc % G;

    int n_keys, hi, lo = 0, wrap_base = 0, pos0 = 0;
    uint32_t rs, kv_bytes;
    const bf16 *kbase, *vbase;
    if (RING) {
        const int L = cache_len ? cache_len[b] : W;
        wrap_base = (L - 1) % W;                             // slot of the newest token
        pos0 = L - 1 - wrap_base;                            // position of slot 0 (before wrap)
        hi = L - T + t;
        lo = max(max(0, L - W), hi - Wnd + 1);               // in the ring and in the window
        n_keys = W;
        rs = (uint32_t)D * 2;
        kbase = kc + ((size_t)b * Hkv + g) * (size_t)W * D;
        vbase = vc + ((size_t)b * Hkv + g) * (size_t)W * D;
        kv_bytes = (uint32_t)W * rs;
    } else {
        const int k_begin = split * kps;
        n_keys = min(S_kv, k_begin + kps) - k_begin;
        pos0 = k_begin;
        hi = S_kv - T + t;
        rs = (uint32_t)Hkv * D * 2;
        kbase = kc + (((size_t)b * S_kv + k_begin) * Hkv + g) * D;
        vbase = vc + (((size_t)b * S_kv + k_begin) * Hkv + g) * D;
        kv_bytes = (uint32_t)(n_keys - 1) * rs + D * 2;
    }
    const rsrc_t kr = make_rsrc(kbase, kv_bytes);            // keys past the item read zeros
    const rsrc_t vr = make_rsrc(vbase, kv_bytes);
    const int n_chunks = (n_keys + kChunk - 1) / kChunk;

    // Q fragments (B operand of S^T): lane half hl feeds dims [D/2*hl, D/2*hl + D/2).
    bf16x8 qf[KF];
    {
        const bf16 *qrow = q + (((size_t)b * T + t) * Hq + h) * D + (D / 2) * hl;
#pragma unroll
        for (int ks = 0; ks < KF; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 8 * ks);
    }
    // K is loaded whole rows at a time (16 lanes per 256-byte row, so every
    // load instruction covers full cache lines; K and V are read once, so the
    // loads are non-temporal) and turned into MFMA
    // fragments through the wave's LDS tile.  Load u, lane i: 16-byte piece
    // e = 64u + i of the chunk, row e / (D/8), column piece e % (D/8).
    bf16x8 kf[KF];                                   // K rows (16-byte pieces) of the current chunk
    bf16x8 vq[VPT][4];                               // V rows (4 keys x 8 dims) of the current chunk
    auto load_k = [&](int k0) {
#pragma unroll
        for (int u = 0; u < KF; ++u) {
            const int e = 64 * u + lane;
            kf[u] = buf_load16_nt(kr, (e / (D / 8)) * rs + 16 * (e % (D / 8)), (uint32_t)k0 * rs);
        }
    };
    auto load_v = [&](int k0) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int it = lane + 64 * i, kq = it & 7, ch = it >> 3;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                vq[i][j] = buf_load16_nt(vr, (4 * kq + j) * rs + 16 * ch, (uint32_t)k0 * rs);
        }
    };

    float m = -INFINITY;                              // running max (log2 units)
    const float s2 = sink[h] * kLog2e;
    if (RING) m = s2;                                 // sink-seeded
    float l = 0.0f;                                   // this lane's share of the real-token sum
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();

    // Each register set is refilled with the next chunk as soon as this
    // chunk has consumed it, so the loads overlap the softmax and PV work.
    // The refill is unconditional: past the item's keys the loads are out
    // of the descriptor's range and return zeros without touching memory.
    // K before V everywhere, so that the S^T products wait only for K.
    // Neighbouring waves start at different chunks of their keys (the order
    // of the chunks does not matter to the online softmax), so that the
    // requests in flight at any moment spread over more address offsets.
    const int rot = n_chunks > 0 ? item % n_chunks : 0;
    load_k(kChunk * rot);
    __builtin_amdgcn_sched_barrier(0);
    load_v(kChunk * rot);
    for (int ci = 0; ci < n_chunks; ++ci) {
        const int cc = ci + rot < n_chunks ? ci + rot : ci + rot - n_chunks;
        const int k0 = kChunk * cc;
        // The next chunk; after the last, an offset past the item's keys
        // (the loads then return zeros without touching memory).
        const int cn = ci + 1 == n_chunks ? n_chunks : (cc + 1 < n_chunks ? cc + 1 : 0);

        // Stage this chunk: K rows as they are, V transposed.  The previous
        // chunk's PV products may still be running, so lds_settle holds the
        // write data registers until the writes are done; then the same
        // registers take the next chunk's loads, which stay in flight for
        // the whole of this chunk's compute.
#pragma unroll
        for (int u = 0; u < KF; ++u) {
            const int e = 64 * u + lane;
            *(bf16x8 *)&kt[e / (D / 8)][8 * (e % (D / 8))] = kf[u];
        }
        lds_settle(kf);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int it = lane + 64 * i, kq = it & 7, ch = it >> 3;
            u32x2 w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x4 x;
                x[0] = vq[i][0][e];
                x[1] = vq[i][1][e];
                x[2] = vq[i][2][e];
                x[3] = vq[i][3][e];
                w[e] = __builtin_bit_cast(u32x2, x);
                *(u32x2 *)&vt[8 * ch + e][4 * kq] = w[e];
            }
            lds_settle(w);
        }
        load_k(kChunk * cn);
        load_v(kChunk * cn);

        // S^T = K Q^T: A row lq is key score_row_key(lq), lane half hl
        // feeds dims [D/2*hl, D/2*hl + D/2) like the Q fragments.
        const bf16 *krow = &kt[score_row_key(lq)][(D / 2) * hl];
        f32x16 sc = mfma32(*(const bf16x8 *)krow, qf[0], zero16());
#pragma unroll
        for (int ks = 1; ks < KF; ++ks) sc = mfma32(*(const bf16x8 *)(krow + 8 * ks), qf[ks], sc);

        // Visibility mask and chunk max.
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = k0 + score_reg_key(r, lane);
            int pos = pos0 + j;
            if (RING && j > wrap_base) pos -= W;
            const bool ok = j < n_keys && pos >= lo && pos <= hi;
            sc[r] = ok ? sc[r] : -INFINITY;
            mx = fmaxf(mx, sc[r]);
        }
        mx = wave_xor32_max(mx) * c;
        if (__ballot(mx > m + kSlack) != 0) {
            const float m_new = fmaxf(m, mx);
            const float alpha = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
            m = m_new;
        }
        const float mu = m == -INFINITY ? 0.0f : m;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mu));
            sc[r] = p;
            l += p;
        }
        const bf16x8 p0 = pack8(sc, 0), p1 = pack8(sc, 1);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            o[dt] = mfma32(*(const bf16x8 *)&vt[32 * dt + lq][8 * hl], p0, o[dt]);
            o[dt] = mfma32(*(const bf16x8 *)&vt[32 * dt + lq][16 + 8 * hl], p1, o[dt]);
        }
    }

    const float mu = m == -INFINITY ? 0.0f : m;
    const float lsum = wave_xor32_sum(l);
    if (RING) {
        // The sink joins the denominator once: l = sum_j e^{x_j - m} + e^{s_h - m}.
        const float lt = lsum + __builtin_amdgcn_exp2f(s2 - mu);
        const float inv = lt > 0.0f ? __builtin_amdgcn_rcpf(lt) : 0.0f;
        // out^T goes through the wave's K tile (free after the last S^T) so
        // that the stores are whole 256-byte rows, 16 bytes per lane.
#pragma unroll
        for (int half = 0; half < D / 64; ++half) {
            u32x2 w[8];
#pragma unroll
            for (int dd = 0; dd < 2; ++dd)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int dt = 2 * half + dd;
                    bf16x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (bf16)(o[dt][4 * jj + e] * inv);
                    w[4 * dd + jj] = __builtin_bit_cast(u32x2, x);
                    *(u32x2 *)&kt[lq][32 * dt + 8 * jj + 4 * hl] = w[4 * dd + jj];
                }
            lds_settle(w);
        }
        constexpr int LPR = D / 8;                    // lanes per output row
#pragma unroll
        for (int r0 = 0; r0 < 32; r0 += 64 / LPR) {
            const int row = r0 + lane / LPR, nr = 32 * ct + row;
            if (nr < G * T) {
                const int tr = nr / G, hr = g * G + nr % G;
                *(bf16x8 *)(out + (((size_t)b * T + tr) * Hq + hr) * D + 8 * (lane % LPR)) =
                    *(const bf16x8 *)&kt[row][8 * (lane % LPR)];
            }
        }
        if (lse != nullptr && hl == 0 && col_ok)
            lse[((size_t)b * Hq + h) * T + t] =
                lt > 0.0f ? (mu + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    } else {
        if (!col_ok) return;
        // partial record [split][b][h][t]: acc[D] (relative to m), then (m, l), log2 units
        const size_t rec = (((size_t)split * B + b) * Hq + h) * T + t;
        float *acc = part + rec * (D + 2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = o[dt][4 * jj + e];
                *(f32x4 *)(acc + 32 * dt + 8 * jj + 4 * hl) = x;
            }
        if (hl == 0) {
            acc[D] = m;
            acc[D + 1] = lsum;
        }
    }
}

// Merge the splits of one (b, h, t) row and add the sink exactly once:
//   M = max(s_h, m_i), l = e^{s_h - M} + sum_i l_i e^{m_i - M},
//   out = sum_i acc_i e^{m_i - M} / l.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const float *__restrict__ part,
                                                     const float *__restrict__ sink,
                                                     bf16 *__restrict__ out, float *__restrict__ lse,
                                                     int B, int Hq, int T, int n_splits) {
    const int lane = threadIdx.x;
    const int row = blockIdx.x;                 // (b, h, t) flattened as [B][Hq][T]
    const int t = row % T, h = (row / T) % Hq, b = row / (T * Hq);
    const size_t stride = (size_t)B * Hq * T * (D + 2);
    const float *base = part + (size_t)row * (D + 2);
    const float s2 = sink[h] * kLog2e;
    float M = s2;
    for (int i = 0; i < n_splits; ++i) M = fmaxf(M, base[i * stride + D]);
    const float Mu = (M == -INFINITY) ? 0.0f : M;
    float l = __builtin_amdgcn_exp2f(s2 - Mu);
    float acc0 = 0.0f, acc1 = 0.0f;
    for (int i = 0; i < n_splits; ++i) {
        const float *p = base + i * stride;
        const float w = p[D + 1] > 0.0f ? __builtin_amdgcn_exp2f(p[D] - Mu) : 0.0f;
        l += p[D + 1] * w;
        acc0 += p[lane] * w;
        if (D > 64) acc1 += p[lane + 64] * w;
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    bf16 *orow = out + (((size_t)b * T + t) * Hq + h) * D;
    orow[lane] = (bf16)(acc0 * inv);
    if (D > 64) orow[lane + 64] = (bf16)(acc1 * inv);
    if (lse != nullptr && lane == 0)
        lse[((size_t)b * Hq + h) * T + t] = l > 0.0f ? (Mu + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
}

int waves_to_groups(long items) { return (int)((items + kWavesPerWG - 1) / kWavesPerWG); }

template <int D>
hipError_t ring_decode_d(const DecodeArgs &a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    const int n_ct = (G * a.T + 31) / 32;
    const long items = (long)n_ct * a.Hkv * a.B;
    hipLaunchKernelGGL((decode_kernel<D, true>), dim3(waves_to_groups(items)), dim3(64 * kWavesPerWG),
                       0, stream, (const bf16 *)a.q, (const bf16 *)a.kcache, (const bf16 *)a.vcache,
                       a.sink, (bf16 *)a.out, a.lse, a.cache_len, a.B, a.Hq, a.Hkv, a.T, a.R, 0, 0,
                       n_ct, 1, (float *)nullptr, a.W);
    return hipGetLastError();
}

// Enough waves to give every SIMD two: each wave streams one key range.
constexpr int kSplitTargetWaves = 2048;

struct SplitPlan {
    int n_splits, kps, n_ct;
};

SplitPlan plan_split(int B, int Hq, int Hkv, int S_q, int S_kv, int D) {
    const int G = Hq / Hkv;
    const int n_ct = (G * S_q + 31) / 32;
    const int ck = kChunk;
    const long pairs = (long)B * Hkv * n_ct;
    const int max_splits = (S_kv + ck - 1) / ck;
    int want = (int)((kSplitTargetWaves + pairs - 1) / pairs);
    want = max(1, min(want, max_splits));
    int kps = (S_kv + want - 1) / want;
    kps = ((kps + ck - 1) / ck) * ck;
    // Each split's buffer window (kps rows of all KV heads) stays below 2^31 bytes.
    const long cap = ((1L << 31) / ((long)Hkv * D * 2)) / ck * ck;
    if (kps > cap) kps = (int)cap;
    const int n_splits = (S_kv + kps - 1) / kps;
    return {n_splits, kps, n_ct};
}

template <int D>
hipError_t splitkv_d(const PrefillArgs &a, void *workspace, hipStream_t stream) {
    const SplitPlan p = plan_split(a.B, a.Hq, a.Hkv, a.S, a.S_kv, a.D);
    float *part = (float *)workspace;
    const long items = (long)p.n_ct * p.n_splits * a.Hkv * a.B;
    hipLaunchKernelGGL((decode_kernel<D, false>), dim3(waves_to_groups(items)),
                       dim3(64 * kWavesPerWG), 0, stream, (const bf16 *)a.q, (const bf16 *)a.k,
                       (const bf16 *)a.v, a.sink, (bf16 *)nullptr, (float *)nullptr,
                       (const int32_t *)nullptr, a.B, a.Hq, a.Hkv, a.S, 0, a.S_kv, p.kps, p.n_ct,
                       p.n_splits, part, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((combine_kernel<D>), dim3(a.B * a.Hq * a.S), dim3(64), 0, stream, part,
                       a.sink, (bf16 *)a.out, a.lse, a.B, a.Hq, a.S, p.n_splits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ring_decode_bf16(const DecodeArgs &a, hipStream_t stream) {
    return a.D == 64 ? ring_decode_d<64>(a, stream) : ring_decode_d<128>(a, stream);
}

int splitkv_num_splits(int B, int Hq, int Hkv, int S_q, int S_kv) {
    return plan_split(B, Hq, Hkv, S_q, S_kv, 128).n_splits;
}

bool splitkv_preferred(int Hq, int Hkv, int S_q, int S_kv) {
    (void)S_kv;
    return (long)(Hq / Hkv) * S_q <= 64;
}

size_t splitkv_workspace_bytes(int B, int Hq, int Hkv, int S_q, int S_kv, int D) {
    const SplitPlan p = plan_split(B, Hq, Hkv, S_q, S_kv, D);
    return (size_t)p.n_splits * B * Hq * S_q * (D + 2) * sizeof(float);
}

hipError_t launch_splitkv_bf16(const PrefillArgs &a, void *workspace, hipStream_t stream) {
    return a.D == 64 ? splitkv_d<64>(a, workspace, stream) : splitkv_d<128>(a, workspace, stream);
}

}  // namespace swa
