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
//  * packed batches of sequences of different lengths (serving mixed
//    context lengths together: "小米罗福莉：MiMo-V2.5如何做到又快又强又便宜？|
//    ICML 2026", §06 Q&A) use the same step code: the concatenation of every
//    sequence's 32-row tiles is split evenly over the work-groups, and a
//    work-group runs one segment per sequence its share meets, each segment
//    starting with its own (window-1)-key halo.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kTile = 32;
constexpr int kMaxTiles = 5;             // ceil((129-1)/32) + 1
constexpr int kRing = kMaxTiles + 1;     // + the tile being prefetched
constexpr int kRingKeys = kRing * kTile;

template <int D, int NW>
struct RingSmem {
    bf16 k[kRing][kTile][D + 8];
    bf16 vt[D][kRingKeys + 8];
    // Per-wave output staging: 32 queries x 64 dims (half of D = 128 at a
    // time), so that global stores are whole 128-byte row segments.
    bf16 ostage[NW][kTile][64 + 8];
};

// Stages one 32-key tile: K rows as 16-byte chunks into sm.k[slot], V as
// 4-key x 8-dim quads written transposed into sm.vt.  The global loads go
// into registers at the start of a step and reach LDS at its end.
template <int D, int NT>
struct Stager {
    static constexpr int CH = D / 8;                       // 16-byte chunks per row
    static constexpr int KPT = (kTile * CH + NT - 1) / NT; // K chunks per thread
    static constexpr int VPT = (8 * CH + NT - 1) / NT;     // V quads per thread
    bf16x8 kreg[KPT];
    bf16x8 vreg[VPT][4];

    // Rows past the end of the descriptor's range read as zeros.
    __device__ __forceinline__ void load(rsrc_t kr, rsrc_t vr, uint32_t rs, uint32_t row0,
                                         int tid) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = min(tid + i * NT, kTile * CH - 1);
            kreg[i] = buf_load16(kr, (item / CH) * rs + 16 * (item % CH), row0 * rs);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int item = min(tid + i * NT, 8 * CH - 1);
            const uint32_t vo = 4 * (item & 7) * rs + 16 * (item >> 3);
#pragma unroll
            for (int j = 0; j < 4; ++j) vreg[i][j] = buf_load16(vr, vo, (row0 + j) * rs);
        }
    }

    template <class Smem>
    __device__ __forceinline__ void store(Smem &sm, int slot, int tid) const {
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

// One work-group = (batch, KV head g, chunk of positions); wave w serves
// query head g*G + w (G = NW waves) for every 32-position step of the chunk.
// Per step and wave the window's key tiles are processed newest first, one
// at a time: S^T = K Q^T (MFMA), band mask on edge tiles, online softmax
// whose running max starts at the sink s_h and is only raised when a tile
// exceeds it by more than 2^8 (so the accumulator is almost never
// rescaled), P packed to bf16, O^T += V^T P^T (MFMA).  The sink adds
// exp(s_h - max) to the denominator once at the end.
//
// Memory pipeline per wave: Q fragments are double-buffered (the loads for
// step n+1 are issued when step n starts), the next step's K/V tile is
// loaded into registers at the start of a step and written into the free
// ring slot at its end, and output stores are never waited on.  Every
// global access is a buffer access relative to this work-group's window of
// the tensor, so rows past the end need no special code.
template <int D, int NW, bool PACKED>
__global__ __launch_bounds__(NW * 64) void swa_prefill_ring_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ sink, bf16 *__restrict__ out, float *__restrict__ lse, int S,
    int Hq, int Hkv, int W, int ntw, int chunk, const int32_t *__restrict__ cu, int B,
    int total) {
    constexpr int NT = NW * 64;
    constexpr float kSlack = 8.0f;                               // log2 units
    constexpr float kBig = 256.0f;                               // 2^kSlack
    __shared__ __align__(16) RingSmem<D, NW> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lq = lane & 31, hl = lane >> 5;
    const int g = blockIdx.y;
    const int h = g * NW + wave;
    const int R = ntw + 1;
    const float c = kLog2e / sqrtf((float)D);
    // key - query for accumulator register r of a tile starting rel keys
    // after the step's first query: 16(r>>3) + (r&7) + kbias + rel
    const int kbias = 8 * hl - lq;
    const uint32_t qrow_bytes = (uint32_t)Hq * D * 2;
    const uint32_t rs = (uint32_t)Hkv * D * 2;

    // The segment being computed: positions [c0, c1) of one sequence.
    // Buffer windows: q/out rows [c0, c1) (all heads); k/v rows [r0, c1) of
    // KV head g -- every row the segment uses (the prefetch past its last
    // tile reads zeros and is never stored); the lse entries of head h.
    int c0 = 0, c1 = 0, r0 = 0;
    rsrc_t qr, orr, kr, vr, lr;
    // QK contraction order: lane half hl feeds dims [64hl, 64hl + 64), the
    // ks-th MFMA step dims 64hl + 8ks .. +8, so each lane reads one whole
    // 128-byte line of its query row (K fragments use the same order).
    const uint32_t q_lane = lq * qrow_bytes + D * hl;              // + 16*ks
    const uint32_t l_lane = hl == 0 ? 4u * lq : kOutOfRange;       // one lane per query
    const float s2 = sink[h] * kLog2e;

    auto load_q = [&](bf16x8 (&qf)[D / 16], int p0) {
        const uint32_t so = (uint32_t)(p0 - c0) * qrow_bytes;    // past the window: zeros
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = buf_load16(qr, q_lane + 16 * ks, so);
    };

    Stager<D, NT> st;

    // S^T of one tile: 32 keys of ring slot `slot` x this wave's 32 queries.
    auto qk = [&](const bf16x8 (&cur)[D / 16], int slot) {
        const bf16 *krow = &sm.k[slot][score_row_key(lq)][(D / 2) * hl];
        f32x16 sc = mfma32(*(const bf16x8 *)krow, cur[0], zero16());
#pragma unroll
        for (int ks = 1; ks < D / 16; ++ks)
            sc = mfma32(*(const bf16x8 *)(krow + 8 * ks), cur[ks], sc);
        return sc;
    };
    // Band mask of a tile starting rel keys after the step's first query.
    auto band = [&](f32x16 &sc, int rel) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dk = 16 * (r >> 3) + (r & 7) + kbias + rel;
            sc[r] = (dk <= 0 && dk > -W) ? sc[r] : -INFINITY;
        }
    };
    // One-sided masks for the steady state: the newest tile only needs
    // key <= query, older tiles only key > query - W (kr <= -kbias and
    // kr > -W - kbias - rel respectively, kr being a per-register constant).
    auto causal = [&](f32x16 &sc) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sc[r] = (16 * (r >> 3) + (r & 7) <= -kbias) ? sc[r] : -INFINITY;
    };
    auto window_edge = [&](f32x16 &sc, int rel) {
        const int thr = -W - kbias - rel;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sc[r] = (16 * (r >> 3) + (r & 7) > thr) ? sc[r] : -INFINITY;
    };
    auto tile_max = [&](const f32x16 &sc) {
        float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sc[r], sc[r + 1]));
        return wave_xor32_max(mx) * c;
    };
    // Raise the running max to cover a tile whose max exceeds it by > slack.
    auto maybe_rescale = [&](float mx, float &m, float &l, f32x16 (&o)[D / 32]) {
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
    };
    // P = exp2(S*c - m) packed to bf16 (two K=16 operands); adds to l.
    // The max is taken on P (canonical exp2 outputs); if some P exceeds
    // 2^slack the running max fell behind: raise it to the tile's exact
    // max, rescale, recompute.  A column whose max is still -inf uses an
    // offset that sends any finite score to +inf.
    auto softmax_tile = [&](f32x16 &sc, float &m, float &l, f32x16 (&o)[D / 32], bf16x8 &p0b,
                            bf16x8 &p1b) {
        f32x16 p;
        {
            const float mu = (m == -INFINITY) ? -3.0e38f : m;
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mu));
        }
        float pm = fmaxf(p[0], p[1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) pm = fmaxf(pm, fmaxf(p[r], p[r + 1]));
        if (__ballot(pm > kBig) != 0) {
            maybe_rescale(tile_max(sc), m, l, o);
            const float mu = (m == -INFINITY) ? -3.0e38f : m;
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mu));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) l += p[r];
        p0b = pack8(p, 0);
        p1b = pack8(p, 1);
    };
    auto pv = [&](f32x16 (&o)[D / 32], const bf16x8 &p0b, const bf16x8 &p1b, int slot) {
        const int col = slot * kTile + 8 * hl;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            o[dt] = mfma32(*(const bf16x8 *)&sm.vt[32 * dt + lq][col], p0b, o[dt]);
            o[dt] = mfma32(*(const bf16x8 *)&sm.vt[32 * dt + lq][col + 16], p1b, o[dt]);
        }
    };

    auto pv_first = [&](f32x16 (&o)[D / 32], const bf16x8 &p0b, const bf16x8 &p1b, int slot) {
        const int col = slot * kTile + 8 * hl;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            o[dt] = mfma32(*(const bf16x8 *)&sm.vt[32 * dt + lq][col], p0b, zero16());
            o[dt] = mfma32(*(const bf16x8 *)&sm.vt[32 * dt + lq][col + 16], p1b, o[dt]);
        }
    };

    // One 32-position step with Q fragments `cur`; refills `fill` with the Q
    // of the next step.
    auto step = [&](const bf16x8 (&cur)[D / 16], bf16x8 (&fill)[D / 16], int p0) {
        const int T1 = p0 / kTile;
        lds_barrier();                                           // ring slot T1 staged
        st.load(kr, vr, rs, kTile * (T1 + 1) - r0, tid);         // next step's tile
        load_q(fill, p0 + kTile);

        float m = s2;                                            // running max (log2 units)
        float l = 0.0f;                                          // this lane's share of sum
        f32x16 o[D / 32];

        // The window is processed newest tile first (98 <= W <= 129: five
        // tiles).  Software-pipelined so the matrix and vector units work at
        // once: the QK products of tile t+1 are issued before the softmax of
        // tile t, the PV products of tile t before the mask/max of tile t+1.
        // Tile 0 needs the causal mask, tile 4 (and tile 3 when W < 128) the
        // window edge; in the first four steps of a sequence, tiles before
        // position 0 read any resident slot and are masked out entirely.
        f32x16 s_cur = qk(cur, T1 % R);
        causal(s_cur);
        m = fmaxf(m, tile_max(s_cur));                           // nothing accumulated yet
#pragma unroll
        for (int t = 0; t < kMaxTiles; ++t) {
            const int T = T1 - t;
            f32x16 s_next;
            if (t + 1 < kMaxTiles) s_next = qk(cur, (T >= 1 ? T - 1 : T1) % R);
            bf16x8 pa, pbb;
            softmax_tile(s_cur, m, l, o, pa, pbb);
            if (t == 0)
                pv_first(o, pa, pbb, T1 % R);
            else
                pv(o, pa, pbb, (T >= 0 ? T : T1) % R);
            if (t + 1 < kMaxTiles) {
                if (T - 1 < 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) s_next[r] = -INFINITY;
                } else if (t + 1 == kMaxTiles - 1 || (t + 1 == kMaxTiles - 2 && W < 4 * kTile)) {
                    window_edge(s_next, -kTile * (t + 1));
                }
                s_cur = s_next;
            }
        }

        // The sink joins the denominator once: l = sum_j e^{x_j - m} + e^{s_h - m}.
        const float mu = (m == -INFINITY) ? 0.0f : m;
        const float lreal = wave_xor32_sum(l);
        l = lreal + __builtin_amdgcn_exp2f(s2 - mu);
        // Epilogue: out = O / l in bf16 (RNE), transposed through this wave's
        // LDS staging area 64 dims at a time and stored as full 128-byte row
        // segments; rows past the window are dropped by the hardware.  The
        // staging writes are issued while the last PV products may still be
        // running, so their data registers are held until they complete.
        // No real-token mass leaves out = 0; every other denominator divides
        // (a NaN one included, so non-finite inputs propagate).
        const float inv = lreal == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(l);
        const uint32_t so = (uint32_t)(p0 - c0) * qrow_bytes;
        bf16 (*stg)[64 + 8] = sm.ostage[wave];
#pragma unroll
        for (int half = 0; half < D / 64; ++half) {
            u32x2 w[8];
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bf16x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (bf16)(o[2 * half + dd][4 * jj + e] * inv);
                    w[4 * dd + jj] = __builtin_bit_cast(u32x2, x);
                    *(u32x2 *)&stg[lq][32 * dd + 8 * jj + 4 * hl] = w[4 * dd + jj];
                }
            }
            lds_settle(w);
            const int ch = lane & 7;
            bf16x8 x[kTile / 8];
#pragma unroll
            for (int i = 0; i < kTile / 8; ++i) x[i] = *(const bf16x8 *)&stg[8 * i + (lane >> 3)][8 * ch];
#pragma unroll
            for (int i = 0; i < kTile / 8; ++i)
                buf_store16_nt(x[i], orr, (8 * i + (lane >> 3)) * qrow_bytes + 128 * half + 16 * ch, so);
            asm volatile("" ::: "memory");             // next half's writes after these reads
        }
        buf_store_f32(l == 0.0f ? -INFINITY : (mu + __builtin_amdgcn_logf(l)) * kLn2, lr, l_lane,
                      (uint32_t)(p0 - c0) * 4);

        if (p0 + kTile < c1) st.store(sm, (T1 + 1) % R, tid);
    };

    // Segments.  Uniform batch (!PACKED): one, the chunk [c0, c1) of
    // sequence blockIdx.z.  Packed batch: sequence s (rows cu[s] .. cu[s+1]-1)
    // contributes ceil(len_s / 32) tiles to one concatenated list, and this
    // work-group owns tiles [t0, t1) of it: a segment per sequence that the
    // range meets.  Each wave finds them with the same scan of 64 sequences
    // at a time (a prefix sum of tile counts), so every value below is
    // wave-uniform and all waves run the same segments.
    const int t0 = blockIdx.x * (chunk / kTile), t1 = t0 + chunk / kTile;
    int sb = 0, carry = 0;                 // next scan batch; tiles before it
    uint64_t pend = 0;                     // lanes of the last batch still to run
    int l_excl = 0, l_n = 0, l_s0 = 0, l_len = 0;
    bool first = true;
    for (;;) {
        size_t row0;
        float *lrow;
        if constexpr (!PACKED) {
            if (!first) break;
            const int b = blockIdx.z;
            row0 = (size_t)b * S;
            c0 = blockIdx.x * chunk;
            c1 = min(S, c0 + chunk);
            lrow = lse != nullptr ? lse + ((size_t)b * Hq + h) * S : nullptr;
        } else {
            while (pend == 0 && sb < B && carry < t1) {
                const int sq = sb + lane;
                int s0 = 0, n_rows = 0;
                if (sq < B) {      // clamped so a malformed table stays inside the tensors
                    s0 = min(max(cu[sq], 0), total);
                    n_rows = min(max(cu[sq + 1], s0), min(total, s0 + S)) - s0;
                }
                const int n = (n_rows + kTile - 1) / kTile;
                int incl = n;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(incl, o);
                    incl += lane >= o ? y : 0;
                }
                l_excl = carry + incl - n;
                l_n = n;
                l_s0 = s0;
                l_len = n_rows;
                pend = __ballot(n > 0 && l_excl < t1 && l_excl + n > t0);
                carry += __builtin_amdgcn_readlane(incl, 63);
                sb += 64;
            }
            if (pend == 0) break;
            const int j = __builtin_ctzll(pend);
            pend &= pend - 1;
            const int excl = __builtin_amdgcn_readlane(l_excl, j);
            const int n = __builtin_amdgcn_readlane(l_n, j);
            const int len = __builtin_amdgcn_readlane(l_len, j);
            row0 = (size_t)__builtin_amdgcn_readlane(l_s0, j);
            c0 = kTile * max(t0 - excl, 0);
            c1 = min(kTile * min(t1 - excl, n), len);
            lrow = lse != nullptr ? lse + (size_t)h * total + row0 : nullptr;
            if (!first) __syncthreads();   // the previous segment's last reads of the ring
        }
        first = false;

        const int T_first = max(0, c0 / kTile - ntw + 1);
        r0 = kTile * T_first;
        qr = make_rsrc(q + ((row0 + c0) * Hq + h) * D, (c1 - c0) * qrow_bytes);
        orr = make_rsrc(out + ((row0 + c0) * Hq + h) * D, (c1 - c0) * qrow_bytes);
        kr = make_rsrc(k + ((row0 + r0) * Hkv + g) * D, (c1 - r0) * rs);
        vr = make_rsrc(v + ((row0 + r0) * Hkv + g) * D, (c1 - r0) * rs);
        lr = make_rsrc(lrow != nullptr ? lrow + c0 : nullptr,
                       lrow != nullptr ? (uint32_t)(c1 - c0) * 4 : 0u);
        bf16x8 qa[D / 16], qb[D / 16];
        if constexpr (!PACKED) {
            // The first step's Q and every window tile up to the step's own
            // are all requested before any is waited for.
            load_q(qa, c0);
            Stager<D, NT> pro[kMaxTiles];
            const int n_pro = c0 / kTile - T_first + 1;   // <= ntw <= kMaxTiles
#pragma unroll
            for (int u = 0; u < kMaxTiles; ++u)
                if (u < n_pro) pro[u].load(kr, vr, rs, kTile * (T_first + u) - r0, tid);
#pragma unroll
            for (int u = 0; u < kMaxTiles; ++u)
                if (u < n_pro) pro[u].store(sm, (T_first + u) % R, tid);
        } else {
            for (int T = T_first; T <= c0 / kTile; ++T) {
                st.load(kr, vr, rs, kTile * T - r0, tid);
                st.store(sm, T % R, tid);
            }
            load_q(qa, c0);
        }
        for (int p0 = c0; p0 < c1; p0 += 2 * kTile) {
            step(qa, qb, p0);
            if (p0 + kTile >= c1) break;
            step(qb, qa, p0 + kTile);
        }
    }
}

}  // namespace

// Largest chunk (a multiple of 32 positions) whose buffer windows stay below
// 2^31 bytes: q/out rows [c0, c1) of all heads, k/v rows [r0, c1) of one KV
// head including the (ntw-1)-tile halo.
int prefill_chunk_cap(int Hq, int Hkv, int D, int ntw) {
    const long limit = 1L << 31;
    const long q_rows = limit / ((long)Hq * D * 2);
    const long kv_rows = limit / ((long)Hkv * D * 2) - (long)kTile * (ntw - 1);
    const long rows = q_rows < kv_rows ? q_rows : kv_rows;
    return (int)(rows < kTile ? kTile : (rows / kTile) * kTile);
}

namespace {

template <int D, int NW>
hipError_t launch_ring(const PrefillArgs &a, hipStream_t stream) {
    const int ntw = (a.window - 1 + kTile - 1) / kTile + 1;
    const int cap_tiles = prefill_chunk_cap(a.Hq, a.Hkv, a.D, ntw) / kTile;
    if (a.cu_seqlens != nullptr) {
        // Packed batch: at most (total + 31 B) / 32 tiles in all; split them
        // evenly over about 256 work-groups (one per CU), at least 4 tiles
        // each so the (ntw-1)-tile halo of a segment stays a small share.
        const long tiles_ub = ((long)a.total + (long)(kTile - 1) * a.B) / kTile;
        long per = (tiles_ub * a.Hkv + 255) / 256;
        per = per < 4 ? 4 : per;
        per = per > cap_tiles ? cap_tiles : per;
        const long nchunks = (tiles_ub + per - 1) / per;
        dim3 grid((unsigned)nchunks, a.Hkv, 1);
        hipLaunchKernelGGL((swa_prefill_ring_kernel<D, NW, true>), grid, dim3(NW * 64), 0, stream,
                           (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.sink,
                           (bf16 *)a.out, a.lse, a.S, a.Hq, a.Hkv, a.window, ntw,
                           (int)per * kTile, a.cu_seqlens, a.B, a.total);
        return hipGetLastError();
    }
    const int tiles = (a.S + kTile - 1) / kTile;
    const int groups = a.B * a.Hkv;
    const int target = 256;                                   // one resident work-group per CU
    int per_group = (target + groups - 1) / groups;
    per_group = max(1, min(per_group, tiles));
    int steps = (tiles + per_group - 1) / per_group;
    steps = max(steps, min(4, tiles));
    const int chunk = min(steps * kTile, cap_tiles * kTile);
    const int nchunks = (a.S + chunk - 1) / chunk;
    dim3 grid(nchunks, a.Hkv, a.B);
    hipLaunchKernelGGL((swa_prefill_ring_kernel<D, NW, false>), grid, dim3(NW * 64), 0, stream,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.sink,
                       (bf16 *)a.out, a.lse, a.S, a.Hq, a.Hkv, a.window, ntw, chunk,
                       (const int32_t *)nullptr, a.B, 0);
    return hipGetLastError();
}

template <int D>
hipError_t launch_ring_d(const PrefillArgs &a, hipStream_t stream) {
    switch (a.Hq / a.Hkv) {          // one wave per query head of the group
    case 1: return launch_ring<D, 1>(a, stream);
    case 2: return launch_ring<D, 2>(a, stream);
    case 4: return launch_ring<D, 4>(a, stream);
    case 8: return launch_ring<D, 8>(a, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace

bool prefill_ring_supported(int window, int G) {
    const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
    return window >= 98 && window <= 129 && g_ok;         // exactly five 32-key tiles
}

hipError_t launch_prefill_ring_bf16(const PrefillArgs &a, hipStream_t stream) {
    return a.D == 64 ? launch_ring_d<64>(a, stream) : launch_ring_d<128>(a, stream);
}

}  // namespace swa
