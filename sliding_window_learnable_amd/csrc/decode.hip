// decode.hip -- short query blocks against a key cache, bf16 MFMA.
//
//  * ring decode: T_q new tokens per sequence against the fixed W-slot
//    sliding-window cache, one work-group per (sequence, KV head), no split
//    (pwwt.cn article on MiMo-V2-Flash, §1.1 Hybrid Attention: the SWA KV
//    cache is fixed-size; technical-report digest, 前置知识 / 多token预测:
//    draft tokens are verified by the main model in one pass).
//  * split-KV partials for global attention over a long linear cache: each
//    work-group reduces one key range to an unnormalised (max, sum, acc)
//    without the sink, and a combine pass merges the splits and adds the
//    sink exactly once (technical-report digest, 前置知识 / 注意力sink偏置).
//
// Columns of the MFMA tiles are (token t, head in group) pairs: G*T_q of
// them per (sequence, KV head), 32 per column tile.  Each wave owns 32 keys
// of a chunk for S^T = K Q^T (K fragments go straight from HBM into the A
// operand registers) and one 32-row d-tile of O^T = V^T P^T; the chunk's V
// is staged transposed in LDS and P is shared through LDS, so the K/V bytes
// of a (sequence, KV head) are read from HBM exactly once for all its heads
// and draft tokens.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

template <int D>
struct DecodeSmem {
    static constexpr int NWD = D / 32;
    static constexpr int CK = 32 * NWD;            // keys per chunk
    bf16 vt[D][CK + 8];
    bf16 pt[32][CK + 8];
    float red_max[NWD][32];
    float red_sum[NWD][32];
};

// Mode RING: keys are ring slots 0..W-1 of [B, Hkv, W, D]; the slot j holds
// position (L-1) - ((L-1-j) mod W), visible to token t when it lies in
// [max(0, L-W), L - T + t].  Mode LINEAR: keys are positions of
// [B, S_kv, Hkv, D] in [split*kps, (split+1)*kps), visible to token t when
// <= S_kv - T + t.
template <int D, bool RING>
__global__ __launch_bounds__(D * 2) void decode_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ kc, const bf16 *__restrict__ vc,
    const float *__restrict__ sink, bf16 *__restrict__ out, float *__restrict__ lse,
    const int32_t *__restrict__ cache_len, int Hq, int Hkv, int T, int W, int S_kv, int kps,
    int n_ct, float *__restrict__ part, int n_splits) {
    constexpr int NWD = D / 32;
    constexpr int CK = 32 * NWD;
    constexpr int NT = 64 * NWD;
    __shared__ __align__(16) DecodeSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lq = lane & 31, hl = lane >> 5;
    const int ct = blockIdx.x % n_ct, split = blockIdx.x / n_ct;
    const int g = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv;
    const float c = kLog2e / sqrtf((float)D);

    // This lane's column: token t, head h.
    const int n = 32 * ct + lq;
    const bool col_ok = n < G * T;
    const int nc = col_ok ? n : 0;
    const int t = nc / G, h = g * G + nc % G;

    long L = 0, lo_pos = 0, hi_pos;     // visible positions for this column
    int k_begin, k_end;                  // key index range of this work-group
    if (RING) {
        L = cache_len ? (long)cache_len[b] : (long)W;
        lo_pos = L - W > 0 ? L - W : 0;
        hi_pos = L - T + t;
        k_begin = 0;
        k_end = W;
    } else {
        hi_pos = (long)S_kv - T + t;
        k_begin = split * kps;
        k_end = min(S_kv, k_begin + kps);
    }

    // Q fragments (B operand of S^T): rows of q [B, T, Hq, D].
    bf16x8 qf[D / 16];
    {
        const bf16 *qrow = q + (((size_t)b * T + t) * Hq + h) * D + 8 * hl;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 16 * ks);
    }

    const bf16 *kbase, *vbase;
    size_t key_stride;
    if (RING) {
        kbase = kc + ((size_t)b * Hkv + g) * (size_t)W * D;
        vbase = vc + ((size_t)b * Hkv + g) * (size_t)W * D;
        key_stride = D;
    } else {
        kbase = kc + ((size_t)b * S_kv * Hkv + g) * D;
        vbase = vc + ((size_t)b * S_kv * Hkv + g) * D;
        key_stride = (size_t)Hkv * D;
    }

    // Running state per column (replicated in every wave).  The ring decode
    // seeds it with the sink: max = s_h, denominator = exp(s_h - s_h) = 1.
    const float s2 = sink[h] * kLog2e;
    float m_run = -INFINITY, l_run = 0.0f;
    if (RING && s2 > -INFINITY) {
        m_run = s2;
        l_run = 1.0f;
    }
    f32x16 o = zero16();

    bf16x8 zero8;
#pragma unroll
    for (int e = 0; e < 8; ++e) zero8[e] = (bf16)0.0f;

    for (int k0 = k_begin; k0 < k_end; k0 += CK) {
        // ---- issue loads: K fragments of this wave's 32 keys, V quads ----
        const int kk = k0 + 32 * wave + score_row_key(lq);
        const bool k_in = kk < k_end;
        const bf16 *krow = kbase + (size_t)(k_in ? kk : k_begin) * key_stride + 8 * hl;
        bf16x8 kf[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) kf[ks] = *(const bf16x8 *)(krow + 16 * ks);

        constexpr int VITEMS = (CK / 4) * (D / 8);
        constexpr int VPT = VITEMS / NT;
        bf16x8 vr[VPT][4];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int item = tid + i * NT;
            const int kq = item % (CK / 4), ch = item / (CK / 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = k0 + 4 * kq + j;
                vr[i][j] = key < k_end
                               ? *(const bf16x8 *)(vbase + (size_t)key * key_stride + 8 * ch)
                               : zero8;
            }
        }

        // ---- S^T for this wave's 32 keys x 32 columns ----
        f32x16 s = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) s = mfma32(kf[ks], qf[ks], s);

        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * wave + score_reg_key(r, lane);
            bool ok = key < k_end;
            if (RING) {
                const long jj = ((L - 1 - key) % W + W) % W;
                const long P = (L - 1) - jj;
                ok = ok && P >= lo_pos && P <= hi_pos;
            } else {
                ok = ok && key <= hi_pos;
            }
            s[r] = ok ? s[r] * c : -INFINITY;
            mx = fmaxf(mx, s[r]);
        }
        mx = wave_xor32_max(mx);

        // ---- stage V^T (transposed) into LDS ----
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int item = tid + i * NT;
            const int kq = item % (CK / 4), ch = item / (CK / 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x4 w;
                w[0] = vr[i][0][e];
                w[1] = vr[i][1][e];
                w[2] = vr[i][2][e];
                w[3] = vr[i][3][e];
                *(bf16x4 *)&sm.vt[8 * ch + e][4 * kq] = w;
            }
        }
        if (hl == 0) sm.red_max[wave][lq] = mx;
        lds_barrier();

        float mc = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWD; ++w) mc = fmaxf(mc, sm.red_max[w][lq]);
        const float m_new = fmaxf(m_run, mc);
        const float mu_new = (m_new == -INFINITY) ? 0.0f : m_new;
        const float mu_old = (m_run == -INFINITY) ? 0.0f : m_run;
        const float alpha = __builtin_amdgcn_exp2f(mu_old - mu_new) * (l_run > 0.0f ? 1.0f : 0.0f);

        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(s[r] - mu_new);
            s[r] = p;
            psum += p;
        }
        psum = wave_xor32_sum(psum);
        *(bf16x8 *)&sm.pt[lq][32 * wave + 8 * hl] = pack8(s, 0);
        *(bf16x8 *)&sm.pt[lq][32 * wave + 16 + 8 * hl] = pack8(s, 1);
        if (hl == 0) sm.red_sum[wave][lq] = psum;
        lds_barrier();

        float lc = 0.0f;
#pragma unroll
        for (int w = 0; w < NWD; ++w) lc += sm.red_sum[w][lq];
        l_run = l_run * alpha + lc;
        m_run = m_new;

        // ---- O^T (d-tile = wave) += V^T P^T over the chunk's keys ----
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] *= alpha;
#pragma unroll
        for (int k16 = 0; k16 < CK / 16; ++k16) {
            const bf16x8 a = *(const bf16x8 *)&sm.vt[32 * wave + lq][16 * k16 + 8 * hl];
            const bf16x8 pb = *(const bf16x8 *)&sm.pt[lq][16 * k16 + 8 * hl];
            o = mfma32(a, pb, o);
        }
        lds_barrier();
    }

    if (!col_ok) return;
    if (RING) {
        const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
        const float mu = (m_run == -INFINITY) ? 0.0f : m_run;
        bf16 *orow = out + (((size_t)b * T + t) * Hq + h) * D + 32 * wave;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (bf16)(o[4 * j + e] * inv);
            *(bf16x4 *)(orow + 8 * j + 4 * hl) = w;
        }
        if (lse != nullptr && wave == 0 && hl == 0)
            lse[((size_t)b * Hq + h) * T + t] =
                l_run > 0.0f ? (mu + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
    } else {
        // partial record [split][b][h][t]: acc[D], then (max, sum) in log2 units
        const int B = gridDim.z;
        const size_t rec = (((size_t)split * B + b) * Hq + h) * T + t;
        float *acc = part + rec * (D + 2) + 32 * wave;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[8 * j + 4 * hl + e] = o[4 * j + e];
        if (wave == 0 && hl == 0) {
            part[rec * (D + 2) + D] = m_run;
            part[rec * (D + 2) + D + 1] = l_run;
        }
    }
    (void)n_splits;
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

template <int D>
hipError_t ring_decode_d(const DecodeArgs &a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    const int n_ct = (G * a.T + 31) / 32;
    dim3 grid(n_ct, a.Hkv, a.B);
    hipLaunchKernelGGL((decode_kernel<D, true>), grid, dim3(D * 2), 0, stream, (const bf16 *)a.q,
                       (const bf16 *)a.kcache, (const bf16 *)a.vcache, a.sink, (bf16 *)a.out,
                       a.lse, a.cache_len, a.Hq, a.Hkv, a.T, a.W, 0, 0, n_ct, (float *)nullptr, 1);
    return hipGetLastError();
}

constexpr int kSplitTargetWGs = 2048;

int chunk_keys(int D) { return D == 64 ? 64 : 128; }

struct SplitPlan {
    int n_splits, kps, n_ct;
};

SplitPlan plan_split(int B, int Hq, int Hkv, int S_q, int S_kv, int D) {
    const int G = Hq / Hkv;
    const int n_ct = (G * S_q + 31) / 32;
    const int ck = chunk_keys(D);
    const long pairs = (long)B * Hkv * n_ct;
    const int max_splits = (S_kv + ck - 1) / ck;
    int want = (int)((kSplitTargetWGs + pairs - 1) / pairs);
    want = max(1, min(want, max_splits));
    int kps = (S_kv + want - 1) / want;
    kps = ((kps + ck - 1) / ck) * ck;
    const int n_splits = (S_kv + kps - 1) / kps;
    return {n_splits, kps, n_ct};
}

template <int D>
hipError_t splitkv_d(const PrefillArgs &a, void *workspace, hipStream_t stream) {
    const SplitPlan p = plan_split(a.B, a.Hq, a.Hkv, a.S, a.S_kv, a.D);
    float *part = (float *)workspace;
    dim3 grid(p.n_splits * p.n_ct, a.Hkv, a.B);
    hipLaunchKernelGGL((decode_kernel<D, false>), grid, dim3(D * 2), 0, stream, (const bf16 *)a.q,
                       (const bf16 *)a.k, (const bf16 *)a.v, a.sink, (bf16 *)nullptr,
                       (float *)nullptr, (const int32_t *)nullptr, a.Hq, a.Hkv, a.S, 0, a.S_kv,
                       p.kps, p.n_ct, part, p.n_splits);
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
