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
//
// Pipeline: key tiles live in an LDS ring of three slots.  At the top of
// iteration t the slots hold tiles t and t+1 and tile t+2 is in flight in
// registers; a wave issues the S^T products of tile t+1 before the softmax
// of tile t (so the matrix unit and the vector unit work at once), then the
// PV products of tile t, then the max of tile t+1.  At the end of the
// iteration tile t+2 is written to the slot freed by tile t-1 and tile t+3
// is requested.  One barrier per tile.  Work-groups are issued longest-first
// (the last query blocks have the most keys) with the (batch, KV head)
// index fastest, so the blocks of one KV head share an XCD and its L2.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kTile = 32;
constexpr int kSlots = 3;
constexpr float kRescaleSlack = 8.0f;    // log2 units
constexpr float kBig = 256.0f;           // 2^kRescaleSlack

template <int D>
struct StreamSmem {
    bf16 k[kSlots][kTile][D + 8];        // row stride 2D+16 bytes: conflict-free fragment reads
    bf16 vt[kSlots][D][kTile + 8];       // V^T, row stride 80 bytes: conflict-free fragment reads
};

// Loads one 32-key tile into registers (K as 16-byte row pieces, V as
// 4-key x 8-dim quads) and writes it to a ring slot, V transposed.  The
// buffer descriptor covers only the tile's rows that exist, so rows past
// the end of the keys read as zeros.
template <int D, int NT>
struct TileLoader {
    static constexpr int CH = D / 8;                       // 16-byte pieces per row
    static constexpr int KPT = (kTile * CH + NT - 1) / NT;
    static constexpr int VPT = (8 * CH + NT - 1) / NT;
    bf16x8 kreg[KPT];
    bf16x8 vreg[VPT][4];

    __device__ __forceinline__ void load(const bf16 *kb, const bf16 *vb, size_t row_elems,
                                         uint32_t rs, int S_kv, int T, int tid) {
        const int rows = min(kTile, S_kv - kTile * T);
        const uint32_t bytes = rows > 0 ? (uint32_t)rows * rs : 0u;
        const rsrc_t kr = make_rsrc(kb + (size_t)kTile * T * row_elems, bytes);
        const rsrc_t vr = make_rsrc(vb + (size_t)kTile * T * row_elems, bytes);
        // Item counts are multiples of 64, so the guards are wave-uniform.
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = tid + i * NT;
            if (item < kTile * CH) kreg[i] = buf_load16(kr, (item / CH) * rs + 16 * (item % CH), 0);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int item = tid + i * NT;
            if (item < 8 * CH) {
                const uint32_t vo = 4 * (item & 7) * rs + 16 * (item >> 3);
#pragma unroll
                for (int j = 0; j < 4; ++j) vreg[i][j] = buf_load16(vr, vo + j * rs, 0);
            }
        }
    }

    __device__ __forceinline__ void store(StreamSmem<D> &sm, int slot, int tid) const {
        if (tid < kTile * CH) {                            // wave-uniform
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int item = tid + i * NT;
                if (item < kTile * CH) *(bf16x8 *)&sm.k[slot][item / CH][8 * (item % CH)] = kreg[i];
            }
            // The data registers take the next tile's loads right after.
            lds_settle(kreg);
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
                // Written while this wave's PV products may still be running.
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
    const int off = S_kv - S_q;                        // row i sits at position off + i
    const int p_first = off + i0;
    const int p_last = off + min(S_q - 1, i0 + kTile - 1);
    const int T_lo = max(0, p_first - W + 1) / kTile;
    const int T_hi = p_last / kTile;
    const int n_tiles = T_hi - T_lo + 1;

    const size_t row_elems = (size_t)Hkv * D;
    const uint32_t rs = (uint32_t)row_elems * 2;
    const bf16 *kb = k + ((size_t)b * S_kv * Hkv + g) * D;
    const bf16 *vb = v + ((size_t)b * S_kv * Hkv + g) * D;

    const int i = i0 + lq;                             // this lane's query row
    const bool row_ok = i < S_q;
    const int pq = off + min(i, S_q - 1);
    // key - query for accumulator register r of tile T:
    //   32T + 16(r>>3) + (r&7) + kbias
    const int kbias = 8 * hl - pq;

    TileLoader<D, NT> ld;
    auto tile_keys_masked = [&](int T) {               // wave-uniform
        return kTile * T + kTile - 1 > p_first || kTile * T <= p_last - W;
    };

    for (int hh = wave; hh < G; hh += NW) {
        const int h = g * G + hh;
        if (hh != wave) lds_barrier();                 // previous head's reads are done
        // Prologue: tiles 0 and 1 into slots 0 and 1, tile 2 in flight.
        ld.load(kb, vb, row_elems, rs, S_kv, T_lo, tid);
        ld.store(sm, 0, tid);
        if (n_tiles > 1) {
            ld.load(kb, vb, row_elems, rs, S_kv, T_lo + 1, tid);
            ld.store(sm, 1, tid);
        }
        if (n_tiles > 2) ld.load(kb, vb, row_elems, rs, S_kv, T_lo + 2, tid);

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

        auto qk = [&](int slot) {
            const bf16 *krow = &sm.k[slot][score_row_key(lq)][8 * hl];
            bf16x8 a[D / 16];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) a[ks] = *(const bf16x8 *)(krow + 16 * ks);
            f32x16 sc = mfma32(a[0], qf[0], zero16());
#pragma unroll
            for (int ks = 1; ks < D / 16; ++ks) sc = mfma32(a[ks], qf[ks], sc);
            return sc;
        };
        auto mask = [&](f32x16 &sc, int T) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dk = kTile * T + 16 * (r >> 3) + (r & 7) + kbias;
                sc[r] = (dk <= 0 && dk > -W) ? sc[r] : -INFINITY;
            }
        };
        auto tile_max = [&](const f32x16 &sc) {
            float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sc[r], sc[r + 1]));
            return wave_xor32_max(mx) * c;
        };
        auto maybe_rescale = [&](float mx) {
            if (__ballot(mx > m + kRescaleSlack) != 0) {
                const float m_new = fmaxf(m, mx);
                const float alpha = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
                m = m_new;
            }
        };

        lds_barrier();                                 // slots 0 and 1 staged
        f32x16 s_cur = qk(0);
        if (tile_keys_masked(T_lo)) mask(s_cur, T_lo);
        // Nothing accumulated yet: the first tile only raises the max.
        m = fmaxf(m, tile_max(s_cur));

        for (int t = 0; t < n_tiles; ++t) {
            const int T = T_lo + t;
            const bool more = t + 1 < n_tiles;
            if (t > 0) lds_barrier();                  // tile t+1 staged, tile t-1 released
            // Past the last tile the product reads a stale slot and is discarded.
            f32x16 s_next = qk((t + 1) % kSlots);

            // P = exp2(S c - m).  The max is taken on P (canonical exp2
            // outputs: max3 without canonicalisation); if some P exceeds
            // 2^slack the running max fell behind: raise it to the tile's
            // exact max, rescale, recompute.  A column whose max is still
            // -inf uses an offset that sends any finite score to +inf.
            f32x16 p;
            {
                const float mu = (m == -INFINITY) ? -3.0e38f : m;
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s_cur[r], c, -mu));
            }
            float pmax = fmaxf(p[0], p[1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) pmax = fmaxf(pmax, fmaxf(p[r], p[r + 1]));
            if (__ballot(pmax > kBig) != 0) {
                maybe_rescale(tile_max(s_cur));
                const float mu = (m == -INFINITY) ? -3.0e38f : m;
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s_cur[r], c, -mu));
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) l += p[r];
            const bf16x8 pa = pack8(p, 0), pb = pack8(p, 1);
            const int slot = t % kSlots;
            bf16x8 va[D / 32][2];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                va[dt][0] = *(const bf16x8 *)&sm.vt[slot][32 * dt + lq][8 * hl];
                va[dt][1] = *(const bf16x8 *)&sm.vt[slot][32 * dt + lq][16 + 8 * hl];
            }
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                o[dt] = mfma32(va[dt][0], pa, o[dt]);
                o[dt] = mfma32(va[dt][1], pb, o[dt]);
            }

            if (more) {
                if (tile_keys_masked(T + 1)) mask(s_next, T + 1);
                s_cur = s_next;
            }
            if (t + 2 < n_tiles) {
                ld.store(sm, (t + 2) % kSlots, tid);
                if (t + 3 < n_tiles) ld.load(kb, vb, row_elems, rs, S_kv, T + 3, tid);
            }
        }

        // Sink joins the denominator once: l_total = sum_j e^{x_j - m} + e^{s_h - m}.
        const float mu = (m == -INFINITY) ? 0.0f : m;
        const float lt = wave_xor32_sum(l) + __builtin_amdgcn_exp2f(s2 - mu);
        if (row_ok) {
            const float inv = lt > 0.0f ? __builtin_amdgcn_rcpf(lt) : 0.0f;
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
