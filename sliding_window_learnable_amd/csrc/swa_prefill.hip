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
//    key tiles T1-4 .. T1 (32 keys each, T1 = the step's own tile), which
//    live in an LDS ring of six tiles -- each step copies ONE new tile, so
//    K and V cross HBM about once plus a (window-1)-key halo per chunk;
//  * per wave and head: S^T = K Q^T on bf16 MFMA tile by tile, band mask on
//    the edge tiles, online softmax seeded with the sink (running max starts
//    at s_h, denominator gets exp(s_h - max) once), O^T = V^T P^T on MFMA,
//    then out = O / l (bf16, RNE) and lse = max + ln l.
//  * packed batches of sequences of different lengths (serving mixed
//    context lengths together: "小米罗福莉：MiMo-V2.5如何做到又快又强又便宜？|
//    ICML 2026", §06 Q&A) use the same step code: the concatenation of every
//    sequence's 32-row tiles is split evenly over the work-groups, and a
//    work-group runs one segment per sequence its share meets, each segment
//    starting with its own (window-1)-key halo.
//
// Memory path: every input reaches LDS by buffer->LDS copies (no staging
// registers): the K and V tiles into the ring, each wave's next 32 query
// rows into its own Q tile, one step ahead (the query rows are read once, in
// whole rows per instruction, so their copies are non-temporal).  The K and
// V ring tiles are interleaved so that each lane reads a tile's fragments
// at one base address plus constants; the Q tiles are unpadded rows whose
// 16-byte chunks are XOR-swizzled by row.  Every fragment read is free of
// bank conflicts.  Once a step's products are issued, the wave moves the next
// step's Q fragments into registers and its Q tile becomes the output
// staging area: the rows of the P.V products are fed dims in the same
// permuted order as the score rows are fed keys, so each lane holds 8
// consecutive dims per register half and writes them as one 16-byte chunk;
// the rows are read back whole and stored as full 256-byte rows per 16
// lanes with non-temporal stores (written once, whole lines reach HBM).
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kTile = 32;
constexpr int kMaxTiles = 5;             // ceil((129-1)/32) + 1
constexpr int kRing = kMaxTiles + 1;     // + the tile being copied

// Ring tiles are interleaved so that every lane reads all its fragments of
// a tile at one base address plus constants (no per-fragment address
// arithmetic) and every read is free of bank conflicts:
//  * K: two groups of 16 rows; row r of a group holds chunk c at
//    16 (r mod 16) + 256 c, so the 16 rows that a 16-byte read serves in
//    one cycle (64 banks) fall on 16 different bank groups, and the chunks
//    a lane reads are 256 bytes apart;
//  * V: blocks of 4 rows, chunk c of row r at 16 (r mod 4) + 64 c, so the
//    32 lanes that an 8-byte transposing read serves in one cycle (4 rows
//    x 4 chunks x 2 halves) fall on 32 different 8-byte bank slots, and the
//    dims a lane reads are 256 bytes per 32 dims apart.
// Each copy instruction fills 1 KiB of a tile, lane l the 16-byte slot l.
template <int D, int NW>
struct RingSmem {
    bf16 k[kRing][kTile][D];             // K tiles, interleaved as above
    bf16 v[kRing][kTile][D];             // V tiles, interleaved as above
    bf16 q[NW][kTile][D];                // each wave's next 32 query rows, swizzled
};

// One work-group = (batch, KV head g, chunk of positions); wave w serves
// query head g*G + w (G = NW waves) for every 32-position step of the chunk.
// Per step and wave the window's key tiles are processed newest first, one
// at a time: S^T = K Q^T (MFMA), band mask on edge tiles, online softmax
// whose running max starts at the sink s_h and is only raised when a tile's
// exponentials sum past 2^8 (so every P stays <= 2^8 and the accumulator is
// almost never rescaled), P packed to bf16, O^T += V^T P^T (MFMA).  The sink adds
// exp(s_h - max) to the denominator once at the end.
//
// Per step n, each wave: passes the work-group barrier (tile T1 is whole --
// every wave waited for its share at the end of step n-1 -- and every wave
// is done with the slot tile T1+1 goes to), starts the copies of tile T1+1
// and of its Q tile for step n+1, computes with the Q fragments of step n,
// waits for those copies, takes the step n+1 fragments into registers,
// stages and stores its output rows.  Every global access is a buffer access relative
// to this work-group's window of the tensor, so rows past the end need no
// special code (loads return zeros, stores are dropped).
template <int D, int NW, bool PACKED>
__global__ __launch_bounds__(NW * 64) void swa_prefill_ring_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ sink, bf16 *__restrict__ out, float *__restrict__ lse, int S,
    int Hq, int Hkv, int W, int ntw, int chunk, const int32_t *__restrict__ cu, int B,
    int total) {
    constexpr float kSlack = 8.0f;                               // log2 units
    constexpr float kBig = 256.0f;                               // 2^kSlack
    constexpr int CPR = D / 8;                                   // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                                // rows per copy instruction
    constexpr int NI = 2 * kTile / RPI;                          // copies per K+V tile
    constexpr int IPW = NI / NW;                                 // ... per wave
    constexpr int QI = kTile / RPI;                              // copies per Q tile
    constexpr int NST = 2 * (D / 32) + 1;                        // stores per step (out, lse)
    static_assert(IPW >= 1 && IPW * NW == NI, "copy split");
    __shared__ __align__(16) RingSmem<D, NW> sm;
    lds_poison_all(sm);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lq = lane & 31, hl = lane >> 5;
    const int g = blockIdx.y;
    const int h = g * NW + wave;
    constexpr int R = kRing;                                     // ntw + 1: the launcher checks
    constexpr uint32_t kTileBytes = kTile * D * 2;
    const float c = kLog2e / sqrtf((float)D);
    // key - query for accumulator register r of a tile starting rel keys
    // after the step's first query: 16(r>>3) + (r&7) + kbias + rel
    const int kbias = 8 * hl - lq;
    const uint32_t qrow_bytes = (uint32_t)Hq * D * 2;
    const uint32_t rs = (uint32_t)Hkv * D * 2;

    // The segment being computed: positions [c0, c1) of one sequence.
    // Buffer windows: q/out rows [c0, c1) (all heads); k/v rows [r0, c1) of
    // KV head g -- every row the segment uses (the copy past its last tile
    // reads zeros and is never used); the lse entries of head h.
    int c0 = 0, c1 = 0, r0 = 0;
    u32x4 qd, kd, vd;
    rsrc_t orr, lr;
    const uint32_t l_lane = hl == 0 ? 4u * lq : kOutOfRange;       // one lane per query
    const float s2 = sink[h] * kLog2e;

    // Copy geometry.  K/V: instruction u of this wave fills 1 KiB (slots
    // 64 iu .. 64 iu + 63) of the K (first half of the instructions) or V
    // tile in the interleaved layouts; Q: instruction u moves rows RPI*u ..
    // of this wave's 32 query rows, lane l's 16 bytes landing at 16*l past
    // the instruction's first row: row l / CPR, chunk position l % CPR,
    // which holds source chunk (l % CPR) ^ swz(row).
    uint32_t kv_off[IPW];
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
        const int ii = wave * IPW + u, sl = 64 * (ii % (NI / 2)) + lane;
        int row, ch;
        if (ii < NI / 2) {                                      // K: groups of 16 rows
            const int w = sl % (16 * CPR);
            row = 16 * (sl / (16 * CPR)) + w % 16;
            ch = w / 16;
        } else {                                                // V: blocks of 4 rows
            const int w = sl % (4 * CPR);
            row = 4 * (sl / (4 * CPR)) + w % 4;
            ch = w / 4;
        }
        kv_off[u] = row * rs + 16 * ch;
    }
    uint32_t q_off[QI];
#pragma unroll
    for (int u = 0; u < QI; ++u) {
        const int row = RPI * u + lane / CPR;
        q_off[u] = row * qrow_bytes + 16 * ((lane % CPR) ^ swz<D>(row));
    }
    // LDS byte addresses of the tiles (uniform).
    const uint32_t k_lds = lds_addr(&sm.k[0][0][0]), v_lds = lds_addr(&sm.v[0][0][0]);
    const uint32_t q_lds = lds_addr(&sm.q[wave][0][0]);
    // Tile T into its ring slot (rows from r0; past the window: zeros).  The
    // tile's offset goes in the copies' scalar offset.
    auto copy_kv = [&](int T) {
        const uint32_t to = (uint32_t)(kTile * T - r0) * rs;
        const uint32_t so = (uint32_t)(T % R) * kTileBytes;
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int ii = wave * IPW + u;                       // uniform
            const bool is_k = ii < NI / 2;
            dma16_at(is_k ? kd : vd, (is_k ? k_lds : v_lds) + so + 1024 * (ii % (NI / 2)), kv_off[u],
                     to);
        }
    };
    // The 32 query rows from position p into this wave's Q tile.
    auto copy_q = [&](int p) {
        const uint32_t to = (uint32_t)(p - c0) * qrow_bytes;
#pragma unroll
        for (int u = 0; u < QI; ++u) dma16_nt_at(qd, q_lds + RPI * u * D * 2, q_off[u], to);
    };

    // QK contraction order: lane half hl feeds dims [D/2*hl, D/2*hl + D/2),
    // the ks-th MFMA step the 16-byte chunk (D/16)*hl + ks -- for the Q
    // fragments (B operand) and the K rows (A operand) alike.
    const int arow = score_row_key(lq);
    const int qrow_s = swz<D>(lq);
    // This lane's K fragments of a tile: row arow, chunks (D/16)*hl + ks at
    // one base plus 256 ks (kept opaque, so that the compiler folds the
    // constants into the reads rather than keeping an address per read).
    uint32_t k_base = k_lds + 32 * D * (arow / 16) + 16 * (arow % 16) + 256 * ((D / 16) * hl);
    asm volatile("" : "+v"(k_base));
    auto read_q = [&](bf16x8 (&qf)[D / 16]) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qf[ks] = *(const bf16x8 *)&sm.q[wave][lq][8 * (((D / 16) * hl + ks) ^ qrow_s)];
    };
    // S^T of one tile: 32 keys of ring slot `slot` x this wave's 32 queries.
    auto qk = [&](const bf16x8 (&cur)[D / 16], int slot) {
        const uint32_t ka = k_base + slot * kTileBytes;
        bf16x8 a[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) a[ks] = lds_read16_at(ka + 256 * ks);
        f32x16 sc = mfma32(a[0], cur[0], zero16());
#pragma unroll
        for (int ks = 1; ks < D / 16; ++ks) sc = mfma32(a[ks], cur[ks], sc);
        // Schedule: four fragment reads ahead of the chained products (left
        // to itself the compiler issues each read right before its product
        // and waits for it: 32K prefill 255.9 -> 250.7 us, same outputs).
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 7);          // LDS reads
#pragma unroll
        for (int ks = 0; ks < D / 16 - 4; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 7);      // a product
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 7);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 7);
        return sc;
    };
    // One-sided masks: the newest tile only needs key <= query, the oldest
    // ones key > query - W (kr <= -kbias and kr > -W - kbias - rel
    // respectively, kr being a per-register constant).
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
    // The check is on the lane's sum of the tile's P (a tree of adds that l
    // needs anyway): every P is >= 0, so a sum within 2^slack bounds each
    // of them; a larger one means the running max may have fallen behind:
    // raise it to the tile's exact max, rescale, recompute.  (A check on
    // the P maximum, 8 more max instructions per tile, measured 1.3% slower
    // at 32K.)  A column whose max is still -inf uses an offset that sends
    // any finite score to +inf.
    auto softmax_tile = [&](f32x16 &sc, float &m, float &l, f32x16 (&o)[D / 32], bf16x8 &p0b,
                            bf16x8 &p1b) {
        f32x16 p;
        {
            const float mu = (m == -INFINITY) ? -3.0e38f : m;
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mu));
        }
        auto tsum = [&]() {
            const float a0 = p[0] + p[1], a1 = p[2] + p[3], a2 = p[4] + p[5], a3 = p[6] + p[7];
            const float a4 = p[8] + p[9], a5 = p[10] + p[11], a6 = p[12] + p[13];
            const float a7 = p[14] + p[15];
            return ((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7));
        };
        float ps = tsum();
        if (__ballot(ps > kBig) != 0) {
            maybe_rescale(tile_max(sc), m, l, o);
            const float mu = (m == -INFINITY) ? -3.0e38f : m;
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mu));
            ps = tsum();
        }
        l += ps;
        p0b = pack8(p, 0);
        p1b = pack8(p, 1);
    };
    // O^T += V^T P^T.  A row m of a 32-dim tile is dim 32dt + score_row_key(m)
    // (the score rows' permutation), so accumulator register r of lane l
    // holds dim 32dt + 16(r>>3) + 8(l>>5) + (r&7): eight consecutive dims per
    // register half.  The A operand comes from the V row tile by transposing
    // reads: in each 16-lane group lane j names 4 dims of key row j/4 --
    // dims 4*pm(j&3) of the group's 16-dim span, pm = (0, 2, 1, 3), which is
    // the permutation within 16 rows -- and lane i receives dim i of the 4 rows.
    // In the V tile (blocks of 4 rows) lane i's rows r1 = 16 kk + 8 hl + tr_j/4
    // and r1 + 4 and its dims 32 dt + tr_d .. + 3 lie at one base plus
    // 32 D kk (16 rows), 8 D (4 rows) and 256 dt (32 dims).
    const int tr_j = lane & 15;
    const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (((tr_j & 1) << 1) | ((tr_j >> 1) & 1));
    uint32_t v_base = v_lds + 16 * D * hl + 16 * (tr_j >> 2) + 64 * (tr_d >> 3) + 8 * ((tr_d >> 2) & 1);
    asm volatile("" : "+v"(v_base));
    auto pv = [&](f32x16 (&o)[D / 32], const bf16x8 &p0b, const bf16x8 &p1b, int slot,
                  bool first) {
        const uint32_t va0 = v_base + slot * kTileBytes;
        bf16x8 va[D / 32][2];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint32_t a = va0 + 256 * dt + 32 * D * kk;
                const bf16x4 lo = lds_read_tr_at(a);
                const bf16x4 hi4 = lds_read_tr_at(a + 8 * D);
                va[dt][kk] = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            o[dt] = mfma32(va[dt][0], p0b, first ? zero16() : o[dt]);
            o[dt] = mfma32(va[dt][1], p1b, o[dt]);
        }
        // Schedule: the transposing reads of two products ahead.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 8);
#pragma unroll
        for (int i = 0; i < D / 16 - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 8);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 8);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 8);
    };

    // Output rows of the previous step, as read back for its stores.  A
    // 16-byte store can read its data registers after the instructions that
    // follow it have already run (later than the compiler's hazard model
    // allows), so these registers are held -- named by the wait that retires
    // the stores -- until the stores are known complete, early in the next
    // step.
    bf16x8 xo[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) xo[i] = bf16x8{};
    bf16x8 cur[D / 16];                  // Q fragments of the current step

    // One 32-position step: Q of this step in `cur`, key tile T1 in the ring
    // (copied during the previous step or the prologue).
    auto step = [&](int p0) {
        const int T1 = p0 / kTile;
        // This wave's share of tile T1 landed before the end of step n-1;
        // after the barrier the whole tile is there and every wave is done
        // with the slot tile T1+1 goes to.
        lds_barrier();
        copy_kv(T1 + 1);                                         // next step's tile
        copy_q(p0 + kTile);                                      // next step's queries
        // The previous step's stores are complete (only this step's copies
        // may be outstanding): their data registers may now be reused.
        hold_until_done<IPW + QI>(xo);

        float m = s2;                                            // running max (log2 units)
        float l = 0.0f;                                          // this lane's share of sum
        f32x16 o[D / 32];

        // The window is processed newest tile first (98 <= W <= 129: five
        // tiles).  Software-pipelined so the matrix and vector units work at
        // once: the QK products of tile t+1 are issued before the softmax of
        // tile t, the PV products of tile t before the mask/max of tile t+1.
        // Tile 0 needs the causal mask, tile 4 (and tile 3 when W < 128) the
        // window edge; in the first four steps of a sequence, tiles before
        // position 0 read the step's own slot and are masked out entirely.
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
            pv(o, pa, pbb, (T >= 0 ? T : T1) % R, t == 0);
            if (t + 1 < kMaxTiles) {
                if (T - 1 < 0) {
                    // A real branch, taken only in a sequence's first four
                    // steps (as selects it costs 16 instructions per tile).
                    asm volatile("" ::: "memory");
#pragma unroll
                    for (int r = 0; r < 16; ++r) s_next[r] = -INFINITY;
                } else if (t + 1 == kMaxTiles - 1 || (t + 1 == kMaxTiles - 2 && W < 4 * kTile)) {
                    window_edge(s_next, -kTile * (t + 1));
                }
                s_cur = s_next;
            }
        }

        // The next step's Q tile has landed (and this step's tile copies):
        // its fragments replace this step's, whose products are all issued.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        read_q(cur);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");       // Q tile free for staging

        // The sink joins the denominator once: l = sum_j e^{x_j - m} + e^{s_h - m}.
        const float mu = (m == -INFINITY) ? 0.0f : m;
        const float lreal = wave_xor32_sum(l);
        l = lreal + __builtin_amdgcn_exp2f(s2 - mu);
        // No real-token mass leaves out = 0; every other denominator divides
        // (a NaN one included, so non-finite inputs propagate).
        const float inv = lreal == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(l);
        // out = O / l in bf16 (RNE): each lane writes its two 8-dim chunks
        // per 32-dim tile into the staging tile (row = its query), then
        // every lane reads back one 16-byte chunk of whole rows and stores
        // it; rows past the window are dropped by the buffer range.  The
        // staging rows rotate their chunks by row (chunk c of row r at
        // c ^ (r % CPR)), not by the operand swizzle: 16-byte LDS writes
        // are served 8 lanes at a time by 32 banks, so the 8 rows of a lane
        // group must land on 8 different chunks modulo 8 (the operand
        // swizzle, built for reads, pairs rows r and r + 2 there and
        // doubled the writes' LDS time).
        const uint32_t so = (uint32_t)(p0 - c0) * qrow_bytes;
        bf16(*stg)[D] = sm.q[wave];
        {
            bf16x8 w[D / 16];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) w[2 * dt + e][i] = (bf16)(o[dt][8 * e + i] * inv);
                    const int ch = (32 * dt + 16 * e + 8 * hl) / 8;
                    *(bf16x8 *)&stg[lq][8 * (ch ^ (lq % CPR))] = w[2 * dt + e];
                }
            lds_settle(w);
        }
#pragma unroll
        for (int u = 0; u < QI; ++u) xo[u] = *(const bf16x8 *)&stg[RPI * u + lane / CPR][8 * (lane % CPR)];
#pragma unroll
        for (int u = 0; u < QI; ++u) {
            const int row = RPI * u + lane / CPR;
            buf_store16_nt(xo[u], orr, row * qrow_bytes + 16 * ((lane % CPR) ^ (row % CPR)), so);
        }
        buf_store_f32(l == 0.0f ? -INFINITY : (mu + __builtin_amdgcn_logf(l)) * kLn2, lr, l_lane,
                      (uint32_t)(p0 - c0) * 4);
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
            // The previous segment's copies have landed and every wave is
            // done reading its ring and Q tiles.
            if (!first) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
            }
        }
        first = false;

        const int T_first = max(0, c0 / kTile - ntw + 1);
        r0 = kTile * T_first;
        qd = sgpr_rsrc(q + ((row0 + c0) * Hq + h) * D, (uint32_t)(c1 - c0) * qrow_bytes);
        kd = sgpr_rsrc(k + ((row0 + r0) * Hkv + g) * D, (uint32_t)(c1 - r0) * rs);
        vd = sgpr_rsrc(v + ((row0 + r0) * Hkv + g) * D, (uint32_t)(c1 - r0) * rs);
        orr = make_rsrc(out + ((row0 + c0) * Hq + h) * D, (c1 - c0) * qrow_bytes);
        lr = make_rsrc(lrow != nullptr ? lrow + c0 : nullptr,
                       lrow != nullptr ? (uint32_t)(c1 - c0) * 4 : 0u);
        // The first step's Q and every window tile up to the step's own are
        // all requested before any is waited for.
        copy_q(c0);
        for (int T = T_first; T <= c0 / kTile; ++T) copy_kv(T);   // <= ntw tiles
        // The first step waits for all of them (no stores are in flight):
        // vmcnt(NST) would leave some copies outstanding, so drain here.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        read_q(cur);
        for (int p0 = c0; p0 < c1; p0 += kTile) step(p0);
    }
    hold_until_done<0>(xo);                                       // nothing left in flight
}

}  // namespace

namespace {

template <int D, int NW>
hipError_t launch_ring(const PrefillArgs &a, hipStream_t stream) {
    const int ntw = (a.window - 1 + kTile - 1) / kTile + 1;
    if (ntw + 1 != kRing) return hipErrorInvalidValue;        // a window of 5 tiles, one more in flight
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

hipError_t launch_prefill_ring_bf16(const PrefillArgs &a, hipStream_t stream) {
    return a.D == 64 ? launch_ring_d<64>(a, stream) : launch_ring_d<128>(a, stream);
}

}  // namespace swa
