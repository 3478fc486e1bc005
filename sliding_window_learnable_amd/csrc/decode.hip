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
// tokens.  Decode is bound by HBM: every wave streams its own keys through
// its own LDS tiles by buffer->LDS copies, the next chunk's copies in flight
// while the current chunk computes, and waves never wait on each other, so
// each CU keeps ~16 KiB per wave in flight.
#include <mutex>

#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kChunk = 32;          // keys per step (one S^T tile)
constexpr int kWavesPerWG = 4;      // independent waves per work-group

// Mode RING: keys are ring slots 0..W-1 of [B, Hkv, W, D]; with base =
// (L-1) mod W the slot j holds position L-1-base+j, minus W when j > base,
// visible to token t when it lies in [max(0, L-W, p-Wnd+1), p], p = L-T+t
// (Wnd: the attention window, at most the W slots).  Mode LINEAR:
// keys are positions [k_begin, k_end) of [B, S_kv, Hkv, D] (one split),
// visible to token t when <= S_kv-T+t.
//
// One wave = one work item (column tile ct, split, KV head g, sequence b):
// it streams the item's keys in 32-key chunks through its own K and V LDS
// tiles.  Per chunk: the K fragments are read once the chunk's K copy has
// landed and the K tile takes the next chunk's copy; S^T = K Q^T, mask,
// online softmax (running max seeded with the sink in RING mode, raised
// lazily); then the V^T fragments (transposing reads) once the V copy has
// landed, the V tile takes the next chunk's copy, and O^T += V^T P^T.  So
// each copy has a whole chunk of compute to land in, and the softmax runs
// while the chunk's V is still arriving.  Waves never synchronise with each
// other.
template <int D, bool RING>
__global__ __launch_bounds__(64 * kWavesPerWG, 2) void decode_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ kc, const bf16 *__restrict__ vc,
    const float *__restrict__ sink, bf16 *__restrict__ out, float *__restrict__ lse,
    const int32_t *__restrict__ cache_len, int B, int Hq, int Hkv, int T, int W, int S_kv,
    int kps, int n_ct, int n_splits, float *__restrict__ part, int Wnd) {
    constexpr int KF = D / 16;                     // Q and K fragments per lane
    constexpr int CPR = D / 8;                     // 16-byte chunks per row
    constexpr int KU = kChunk * D * 2 / 1024;      // copy instructions per tile
    constexpr float kSlack = 8.0f;                 // log2 units
    // Each wave's K and V tiles of one chunk, filled by buffer->LDS copies
    // (lane l of a copy instruction fills the 16-byte slot l of its 1 KiB),
    // each instruction whole rows (whole cache lines).  K: unpadded rows,
    // chunk c of row r at c ^ swz(r); V: blocks of 4 rows, chunk c of row r
    // at 8D (r/4) + 16 (r%4) + 64 c.  The fragment reads (K as rows, V
    // transposed) are free of bank conflicts, and their addresses are the
    // same for every chunk.
    __shared__ __align__(16) bf16 kv_all[kWavesPerWG][2][kChunk][D];

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
    bf16 (*kt)[D] = kv_all[wave][0];              // the K tile, also the output staging area
    lds_poison_wave(kv_all[wave]);
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
        // Until the ring has wrapped (L < W) only slots 0 .. L-1 have been
        // written: the range stops there, so the unwritten slots read as
        // zeros and whatever bits they hold never reach a product (a masked
        // key's zero weight times a non-finite value would still be NaN).
        kv_bytes = (uint32_t)min(max(L, 0), W) * rs;
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
    const u32x4 kr = sgpr_rsrc(kbase, kv_bytes);             // keys past the item read zeros
    const u32x4 vr = sgpr_rsrc(vbase, kv_bytes);
    const int n_chunks = (n_keys + kChunk - 1) / kChunk;

    // Q fragments (B operand of S^T): lane half hl feeds dims [D/2*hl, D/2*hl + D/2).
    bf16x8 qf[KF];
    {
        const bf16 *qrow = q + (((size_t)b * T + t) * Hq + h) * D + (D / 2) * hl;
#pragma unroll
        for (int ks = 0; ks < KF; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 8 * ks);
    }
    // Copy geometry of a chunk: K instruction u moves rows RPI u .. RPI u +
    // RPI - 1, lane l's 16 bytes holding source chunk (l % CPR) ^ swz(row);
    // V instruction u fills slots 64 u .. 64 u + 63 of the V tile (64/CPR
    // rows), the source offset a per-lane part plus a uniform one.  Whole
    // cache lines are read per instruction (both are read once: the copies
    // are non-temporal).
    constexpr int RPI = 64 / CPR;                  // K rows per copy instruction
    const uint32_t v_lane = (4 * (lane / (4 * CPR)) + lane % 4) * rs + 16 * ((lane % (4 * CPR)) / 4);
    const uint32_t k_lds = lds_addr(&kv_all[wave][0][0][0]), v_lds = lds_addr(&kv_all[wave][1][0][0]);
    auto copy_k = [&](int k0) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = RPI * u + lane / CPR;
            dma16_nt_at(kr, k_lds + 1024 * u, row * rs + 16 * ((lane % CPR) ^ swz<D>(row)),
                        (uint32_t)k0 * rs);
        }
    };
    auto copy_v = [&](int k0) {
#pragma unroll
        for (int u = 0; u < KU; ++u)
            dma16_nt_at(vr, v_lds + 1024 * u, v_lane, (uint32_t)(k0 + (64 / CPR) * u) * rs);
    };
    // Fragment addresses: K row score_row_key(lq), chunks (D/16) hl + ks;
    // V^T rows r1 = 16 kk + 8 hl + tr_j/4 and r1 + 4,
    // dims 32 dt + tr_d .. + 3, at one base plus 32 D kk, 8 D and 256 dt.
    const int arow = score_row_key(lq);
    const int tr_j = lane & 15, tr_d = 16 * ((lane >> 4) & 1) + 4 * (tr_j & 3);
    uint32_t v_base = v_lds + 16 * D * hl + 16 * (tr_j >> 2) + 64 * (tr_d >> 3) + 8 * ((tr_d >> 2) & 1);
    asm volatile("" : "+v"(v_base));

    float m = -INFINITY;                              // running max (log2 units)
    const float s2 = sink[h] * kLog2e;
    // Sink-seeded; a NaN sink is left out of the max so that it reaches the
    // results only through the denominator (as in the definition: a row
    // with no visible key then keeps out = 0, and lse becomes NaN).
    if (RING && !__builtin_isnan(s2)) m = s2;
    float l = 0.0f;                                   // this lane's share of the real-token sum
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();

    // Each chunk's fragments are read into registers as soon as it has
    // landed; then the next chunk's copies go to the same tiles, in flight
    // for the whole of this chunk's compute.  Neighbouring waves start at
    // different chunks of their keys (the order of the chunks does not
    // matter to the online softmax), so that the requests in flight at any
    // moment spread over more address offsets.
    const int rot = n_chunks > 0 ? item % n_chunks : 0;
    if (n_chunks > 0) {
        copy_k(kChunk * rot);
        copy_v(kChunk * rot);
    }
    for (int ci = 0; ci < n_chunks; ++ci) {
        const int cc = ci + rot < n_chunks ? ci + rot : ci + rot - n_chunks;
        const int k0 = kChunk * cc;
        const int cn = cc + 1 < n_chunks ? cc + 1 : 0;

        const bool more = ci + 1 < n_chunks;                        // uniform
        // K of this chunk landed (its V may still be in flight): read the
        // K fragments, then the K tile takes the next chunk's copy.
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KU) : "memory");
        bf16x8 kf[KF], va[D / 32][2];
#pragma unroll
        for (int ks = 0; ks < KF; ++ks)
            kf[ks] = *(const bf16x8 *)&kt[arow][8 * (((D / 16) * hl + ks) ^ swz<D>(arow))];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (more) copy_k(kChunk * cn);

        // S^T = K Q^T: A row lq is key score_row_key(lq), lane half hl
        // feeds dims [D/2*hl, D/2*hl + D/2) like the Q fragments.
        f32x16 sc = mfma32(kf[0], qf[0], zero16());
#pragma unroll
        for (int ks = 1; ks < KF; ++ks) sc = mfma32(kf[ks], qf[ks], sc);

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
        // This chunk's V landed (only the next chunk's K copies may be
        // outstanding): read the V^T fragments, then the V tile takes the
        // next chunk's copy.
        if (more) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KU) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint32_t a = v_base + 256 * dt + 32 * D * kk;
                const bf16x4 lo = lds_read_tr_at(a), hi4 = lds_read_tr_at(a + 8 * D);
                va[dt][kk] = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (more) copy_v(kChunk * cn);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            o[dt] = mfma32(va[dt][0], p0, o[dt]);
            o[dt] = mfma32(va[dt][1], p1, o[dt]);
        }
    }

    const float mu = m == -INFINITY ? 0.0f : m;
    const float lsum = wave_xor32_sum(l);
    if (RING) {
        // The sink joins the denominator once: l = sum_j e^{x_j - m} + e^{s_h - m}.
        // No real-token mass (no visible key) leaves out = 0; any other
        // denominator, NaN included, divides, so non-finite inputs propagate.
        const float lt = lsum + __builtin_amdgcn_exp2f(s2 - mu);
        const float inv = lsum == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(lt);
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
                lt == 0.0f ? -INFINITY : (mu + __builtin_amdgcn_logf(lt)) * kLn2;
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
    float lreal = 0.0f;                         // real-token mass
    float acc0 = 0.0f, acc1 = 0.0f;
    for (int i = 0; i < n_splits; ++i) {
        const float *p = base + i * stride;
        // a split that saw nothing has l = 0 (and m = -inf): weight 0; a NaN
        // l also gets weight 0 and still turns the sums into NaN
        const float w = p[D + 1] > 0.0f ? __builtin_amdgcn_exp2f(p[D] - Mu) : 0.0f;
        lreal += p[D + 1] * w;
        acc0 += p[lane] * w;
        if (D > 64) acc1 += p[lane + 64] * w;
    }
    const float l = lreal + __builtin_amdgcn_exp2f(s2 - Mu);
    const float inv = lreal == 0.0f ? 0.0f : 1.0f / l;
    bf16 *orow = out + (((size_t)b * T + t) * Hq + h) * D;
    orow[lane] = (bf16)(acc0 * inv);
    if (D > 64) orow[lane + 64] = (bf16)(acc1 * inv);
    if (lse != nullptr && lane == 0)
        lse[((size_t)b * Hq + h) * T + t] = l == 0.0f ? -INFINITY : (Mu + __builtin_amdgcn_logf(l)) * kLn2;
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

hipError_t launch_splitkv_bf16(const PrefillArgs &a, void *workspace, hipStream_t stream) {
    return a.D == 64 ? splitkv_d<64>(a, workspace, stream) : splitkv_d<128>(a, workspace, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the split-KV partials go to a static device array
// instead of a caller workspace.  Each GPU holds its own copy of `scratch`
// for the life of the process; host code only ever passes the device address
// found by hipGetSymbolAddress (once per device, with that device current).
// Every record the combine pass reads is written by the partial pass of the
// same call, so nothing in it has to start at zero.  Calls that overlap on
// one GPU (several streams or host threads) share the array and race.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_splitkv_bf16_static(const PrefillArgs &a, hipStream_t stream) {
    void *ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    return launch_splitkv_bf16(a, ws, stream);
}

}  // namespace swa
