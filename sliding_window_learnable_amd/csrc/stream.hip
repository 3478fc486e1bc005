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
//   rescaling (the accumulator is rescaled only when a tile's exponentials
//   sum past 2^8 in some column, so every exp2 argument stays <= 8),
//   O^T += V^T P^T (bf16 MFMA).
// At the end the sink's exp(s_h - max) joins the denominator exactly once.
//
// Pipeline: key tiles are copied from memory straight into an LDS ring of
// four slots (buffer->LDS copies, no staging registers), three tiles ahead,
// interleaved so that a lane reads all its fragments of a tile at one base
// address plus constants, free of bank conflicts: K rows feed the A operand
// of S^T directly and V^T is read with transposing LDS reads.  In
// iteration t a wave issues the S^T products of tile t+1 before the
// softmax of tile t (so the matrix unit and the vector unit work at once),
// then the PV products of tile t; the copies of tile t+3 go to the slot
// tile t-1 freed.  One barrier per tile.
//
// Work order: the KV head index is the fastest (consecutive work-groups go
// to different XCDs, so the blocks of one KV head share an XCD and its
// L2), then the query blocks of one sequence, longest first (the last
// query blocks have the most keys), then the sequences.  So the
// work-groups that run together on an XCD mostly belong to one sequence
// and read the same key tiles through its L2; taken in query-block order
// across the batch, the 32 or so resident work-groups of an XCD would
// belong to as many sequences as the batch holds and share almost nothing.
// Packed batches of sequences of different lengths: sequence s owns the
// 32-row slots j with 32j in [cu[s] + 32s, cu[s+1] + 32(s+1)), at least
// ceil(len_s / 32) of them, with no table built on the host; a work-group
// finds its sequence by a 64-way search of cu and returns before touching
// memory or a barrier when its slot is a spare one.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kTile = 32;
constexpr int kSlots = 4;
constexpr float kRescaleSlack = 8.0f;    // log2 units
constexpr float kBig = 256.0f;           // 2^kRescaleSlack

// K tiles: two groups of 16 rows, row r of a group holding chunk c at
// 16 (r mod 16) + 256 c.  V tiles: blocks of 4 rows, chunk c of row r at
// 16 (r mod 4) + 64 c.  Each copy instruction fills 1 KiB of a tile,
// lane l the 16-byte slot l.
template <int D>
struct StreamSmem {
    bf16 k[kSlots][kTile][D];            // K tiles, interleaved as above
    bf16 v[kSlots][kTile][D];            // V tiles, interleaved as above
};

// BLK: also write, per (query head, 32-row block, key block of 32 rk keys),
// the largest scaled logit q.k/sqrt(D) over the block's visible pairs
// (-inf when none) to bmax [B, Hq, NB, NKB].  The max is taken on the
// softmax's own exponent arguments t = s c - m (one v_max per score, no
// canonicalisation), m added back per tile; each lane keeps a running max
// over the tiles of the current key block, reduced across the wave once
// per key block.
template <int D, int NW, bool BLK>
__global__ __launch_bounds__(NW * 64) void stream_attn_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ sink, bf16 *__restrict__ out, float *__restrict__ lse, int S_q_,
    int S_kv_, int Hq, int Hkv, int W, int BG, int NB, float *__restrict__ bmax, int rk, int NKB,
    const int32_t *__restrict__ cu, int total) {
    __shared__ __align__(16) StreamSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lq = lane & 31, hl = lane >> 5;
    const int G = Hq / Hkv;
    const float c = kLog2e / sqrtf((float)D);

    // Packed variable-length batch (cu != nullptr): sequence b owns rows
    // cu[b] .. cu[b+1]-1 of [total, H, D] tensors (lse [Hq, total]) and
    // attends within itself; otherwise [B, S, H, D] (lse [B, Hq, S_q]).
    int S_q = S_q_, S_kv = S_kv_, b, g, qb;
    size_t q_row0, kv_row0;
    if (cu == nullptr) {
        g = blockIdx.x % Hkv;
        const int j = blockIdx.x / Hkv;
        b = j / NB;
        qb = NB - 1 - j % NB;                          // longest query blocks first
        q_row0 = (size_t)b * S_q_;
        kv_row0 = (size_t)b * S_kv_;
    } else {
        // Table values are clamped to [0, total] throughout, so a malformed
        // table cannot index past the tensors (nor stop the search).
        const int B = BG / Hkv;                        // sequences
        g = blockIdx.x % Hkv;
        const long slot = (long)(blockIdx.x / Hkv) * kTile;
        auto start = [&](int s) {                      // 32s + cu[s], clamped
            return (long)kTile * s + min(max(cu[s], 0), total);
        };
        if (start(0) > slot) return;
        int lo = 0, hi = B;                            // start(lo) <= slot
        while (hi - lo > 1) {                          // wave-uniform
            const int step = (hi - lo + 63) / 64, s = lo + lane * step;
            const uint64_t ok = __ballot(s < hi && start(min(s, B)) <= slot);
            const int last = 63 - __builtin_clzll(ok);  // lane 0 (s = lo) always passes
            lo += last * step;
            hi = min(hi, lo + step);
        }
        b = lo;
        const int s0 = min(max(cu[b], 0), total);
        const int s1 = min(max(cu[b + 1], s0), min(total, s0 + S_q_));
        S_q = S_kv = s1 - s0;
        q_row0 = kv_row0 = (size_t)s0;
        const long first = (start(b) + kTile - 1) / kTile;   // the sequence's first slot
        qb = (S_q + kTile - 1) / kTile - 1 - (int)(slot / kTile - first);   // longest first
        if (qb < 0) return;                            // a spare slot (uniform, before any barrier)
    }
    const int i0 = qb * kTile;                         // first query row of the block
    if (i0 >= S_q) return;                             // past this sequence (uniform, before any barrier)
    lds_poison_all(sm);
    const int off = S_kv - S_q;                        // row i sits at position off + i
    const int p_first = off + i0;
    const int p_last = off + min(S_q - 1, i0 + kTile - 1);
    const int T_lo = max(0, p_first - W + 1) / kTile;
    const int T_hi = p_last / kTile;
    const int n_tiles = T_hi - T_lo + 1;

    const size_t row_elems = (size_t)Hkv * D;
    const uint32_t rs = (uint32_t)row_elems * 2;
    const bf16 *kb = k + (kv_row0 * Hkv + g) * D;
    const bf16 *vb = v + (kv_row0 * Hkv + g) * D;

    const int i = i0 + lq;                             // this lane's query row
    const bool row_ok = i < S_q;
    const int pq = off + min(i, S_q - 1);
    // key - query for accumulator register r of tile T:
    //   32T + 16(r>>3) + (r&7) + kbias
    const int kbias = 8 * hl - pq;

    auto tile_keys_masked = [&](int T) {               // wave-uniform
        return kTile * T + kTile - 1 > p_first || kTile * T <= p_last - W;
    };
    // Copies of one tile: 2 * 32 rows of 2D bytes in 1 KB instructions, IPW
    // per wave (K first, then V); rows past the end of the keys land as zero.
    constexpr int CPR = D / 8;                         // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                      // rows per instruction
    constexpr int NI = 2 * kTile / RPI;                // instructions per tile
    constexpr int IPW = NI / NW;
    static_assert(IPW >= 1 && IPW * NW == NI, "copy split");
    constexpr uint32_t kTileBytes = kTile * D * 2;
    uint32_t dma_off[IPW];
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
        const int ii = wave * IPW + u, sl = 64 * (ii % (NI / 2)) + lane;
        int row, ch;
        if (ii < NI / 2) {                             // K: groups of 16 rows
            const int w = sl % (16 * CPR);
            row = 16 * (sl / (16 * CPR)) + w % 16;
            ch = w / 16;
        } else {                                       // V: blocks of 4 rows
            const int w = sl % (4 * CPR);
            row = 4 * (sl / (4 * CPR)) + w % 4;
            ch = w / 4;
        }
        dma_off[u] = row * rs + 16 * ch;
    }
    const uint32_t k_lds = lds_addr(&sm.k[0][0][0]), v_lds = lds_addr(&sm.v[0][0][0]);
    // When the whole key range of the sequence fits one descriptor's 32-bit
    // range, the descriptors are built once and a tile's offset rides in the
    // per-lane offset (range-checked, so rows past the end still land as
    // zero); otherwise each tile gets descriptors of its own.
    const bool one_rsrc = (unsigned long long)(S_kv + kTile) * rs <= (1ull << 32);   // no offset wraps
    const uint32_t seq_bytes = one_rsrc && S_kv > 0 ? (uint32_t)(S_kv - 1) * rs + D * 2 : 0u;
    const u32x4 k_all = sgpr_rsrc(kb, seq_bytes), v_all = sgpr_rsrc(vb, seq_bytes);
    auto stage = [&](int T, int slot) {
        u32x4 kr = k_all, vr = v_all;
        uint32_t to_b = (uint32_t)(kTile * T) * rs;
        if (!one_rsrc) {
            const int rows = min(kTile, S_kv - kTile * T);
            const uint32_t bytes = rows > 0 ? (uint32_t)(rows - 1) * rs + D * 2 : 0u;
            const size_t to = (size_t)kTile * T * row_elems;
            kr = sgpr_rsrc(kb + to, bytes);
            vr = sgpr_rsrc(vb + to, bytes);
            to_b = 0;
        }
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int ii = wave * IPW + u;             // uniform
            const bool is_k = ii < NI / 2;
            dma16_at(is_k ? kr : vr,
                     (is_k ? k_lds : v_lds) + slot * kTileBytes + 1024 * (ii % (NI / 2)), dma_off[u],
                     to_b);
        }
    };
    auto dma_wait = [&](bool newer) {
        if (newer) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // This lane's fragment addresses in ring slot 0 (opaque, so that the
    // constants stay immediates of the reads): K row score_row_key(lq),
    // chunks 2 ks + hl at one base plus 512 ks; V^T rows r1 = 16 kk + 8 hl +
    // tr_j/4 and r1 + 4, dims 32 dt + tr_d .. + 3, at one base plus 32 D kk,
    // 8 D and 256 dt.
    const int arow_r = score_row_key(lq);
    const int tr_j = lane & 15, tr_d = 16 * ((lane >> 4) & 1) + 4 * (tr_j & 3);
    uint32_t k_base, v_base;
    {
        k_base = k_lds + 32 * D * (arow_r / 16) + 16 * (arow_r % 16) + 256 * hl;
        v_base = v_lds + 16 * D * hl + 16 * (tr_j >> 2) + 64 * (tr_d >> 3) + 8 * ((tr_d >> 2) & 1);
        asm volatile("" : "+v"(k_base), "+v"(v_base));
    }

    for (int hh = wave; hh < G; hh += NW) {
        const int h = g * G + hh;
        if (hh != wave) lds_barrier();                 // previous head's reads are done
        // Tiles 0, 1 (and 2, left in flight) start copying into slots 0, 1, 2
        // before the Q loads, so the two latencies overlap.
        for (int t = 0; t < 3 && t < n_tiles; ++t) stage(T_lo + t, t);
        bf16x8 qf[D / 16];
        {
            const bf16 *qrow = q + ((q_row0 + min(i, S_q - 1)) * Hq + h) * D + 8 * hl;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 16 * ks);
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) retire(qf[ks]);
        }
        if (n_tiles > 2) dma_wait(true);
        else dma_wait(false);
        const float s2 = sink[h] * kLog2e;
        float m = s2;                                  // running max seeded with the sink
        float l = 0.0f;                                // this lane's share of the real-token sum
        f32x16 o[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();

        auto qk = [&](int slot) {
            const uint32_t ka = k_base + slot * kTileBytes;
            bf16x8 a[D / 16];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) a[ks] = lds_read16_at(ka + 512 * ks);
            f32x16 sc = mfma32(a[0], qf[0], zero16());
#pragma unroll
            for (int ks = 1; ks < D / 16; ++ks) sc = mfma32(a[ks], qf[ks], sc);
            // Schedule: two fragment reads ahead of the chained products
            // (64K global layer 67.13 -> 66.15 ms with the P.V schedule
            // below; deeper read-ahead measured no better).
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 7);      // LDS reads
#pragma unroll
            for (int ks = 0; ks < D / 16 - 2; ++ks) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 7);  // a product
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 7);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 7);
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

        // Block maxima: running max of the raw scores of this lane, per key block.
        float bm_run = -INFINITY;
        float *brow = BLK ? bmax + (((size_t)b * Hq + h) * NB + qb) * NKB : nullptr;
        // tmax: max over this lane's exponent arguments of tile T (log2
        // units, relative to mu); bm_run is kept in absolute log2 units.
        auto block_step = [&](float tmax, float mu, int T) {
            bm_run = fmaxf(bm_run, tmax + mu);
            if ((T + 1) % rk == 0 || T == T_hi) {      // last tile of a key block (uniform)
                float w = bm_run;
#pragma unroll
                for (int sh = 1; sh < 64; sh <<= 1) w = fmaxf(w, __shfl_xor(w, sh));
                if (lane == 0) brow[T / rk] = w == -INFINITY ? -INFINITY : w * kLn2;
                bm_run = -INFINITY;
            }
        };
        if (BLK) {                                     // key blocks past the diagonal see nothing
            for (int kb = T_hi / rk + 1 + lane; kb < NKB; kb += 64) brow[kb] = -INFINITY;
        }

        lds_barrier();                                 // slots 0 and 1 landed
        f32x16 s_cur = qk(0);
        if (tile_keys_masked(T_lo)) mask(s_cur, T_lo);
        // Nothing accumulated yet: the first tile only raises the max.
        m = fmaxf(m, tile_max(s_cur));

        for (int t = 0; t < n_tiles; ++t) {
            const int T = T_lo + t;
            const bool more = t + 1 < n_tiles;
            if (t > 0) lds_barrier();                  // tile t+1 landed, tile t-1 released
            const bool copy = t + 3 < n_tiles;
            if (copy) stage(T + 3, (t + 3) % kSlots);  // into the slot tile t-1 freed
            // Past the last tile the product reads a stale slot and is discarded.
            f32x16 s_next = qk((t + 1) % kSlots);

            // P = exp2(S c - m).  The check is on the lane's sum of the
            // tile's P (a tree of adds that l needs anyway): every P is >= 0,
            // so a sum within 2^slack bounds each of them; a larger one means
            // the running max may have fallen behind: raise it to the tile's
            // exact max, rescale, recompute (a check on the P maximum, 8 more
            // max instructions per tile, measured 1.3% slower at 64K).  A
            // column whose max is still -inf uses an offset that sends any
            // finite score to +inf.
            f32x16 p;
            float tmax = -INFINITY, mu = (m == -INFINITY) ? -3.0e38f : m;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float ta = fmaf(s_cur[r], c, -mu), tb = fmaf(s_cur[r + 1], c, -mu);
                p[r] = __builtin_amdgcn_exp2f(ta);
                p[r + 1] = __builtin_amdgcn_exp2f(tb);
                if (BLK) tmax = fmaxf(tmax, fmaxf(ta, tb));   // v_max3
            }
            auto tsum = [&]() {
                const float a0 = p[0] + p[1], a1 = p[2] + p[3], a2 = p[4] + p[5], a3 = p[6] + p[7];
                const float a4 = p[8] + p[9], a5 = p[10] + p[11], a6 = p[12] + p[13];
                const float a7 = p[14] + p[15];
                return ((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7));
            };
            float ps = tsum();
            if (__ballot(ps > kBig) != 0) {
                maybe_rescale(tile_max(s_cur));
                mu = (m == -INFINITY) ? -3.0e38f : m;
                tmax = -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float ta = fmaf(s_cur[r], c, -mu), tb = fmaf(s_cur[r + 1], c, -mu);
                    p[r] = __builtin_amdgcn_exp2f(ta);
                    p[r + 1] = __builtin_amdgcn_exp2f(tb);
                    if (BLK) tmax = fmaxf(tmax, fmaxf(ta, tb));
                }
                ps = tsum();
            }
            if (BLK) block_step(tmax, mu, T);
            l += ps;
            const bf16x8 pa = pack8(p, 0), pb = pack8(p, 1);
            // O^T += V^T P^T: A row m = dim 32dt + m, k = key 16kk + 8hl + 0..7,
            // from the V row tile by transposing reads of 4 keys each.
            const uint32_t va0 = v_base + (t % kSlots) * kTileBytes;
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
                o[dt] = mfma32(va[dt][0], pa, o[dt]);
                o[dt] = mfma32(va[dt][1], pb, o[dt]);
            }
            // Schedule: the transposing reads of one product ahead.
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 8);
#pragma unroll
            for (int i = 0; i < D / 16 - 1; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 8);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 8);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 8);

            if (more) {
                if (tile_keys_masked(T + 1)) mask(s_next, T + 1);
                s_cur = s_next;
            }
            dma_wait(copy);                            // tile t+2 landed (t+3 may be in flight)
        }

        // Sink joins the denominator once: l_total = sum_j e^{x_j - m} + e^{s_h - m}.
        const float mu = (m == -INFINITY) ? 0.0f : m;
        const float lreal = wave_xor32_sum(l);
        const float lt = lreal + __builtin_amdgcn_exp2f(s2 - mu);
        if (row_ok) {
            // No real-token mass leaves out = 0; every other denominator
            // divides (a NaN one included, so non-finite inputs propagate).
            const float inv = lreal == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(lt);
            bf16 *orow = out + ((q_row0 + i) * Hq + h) * D;
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
                lse[(cu != nullptr ? (size_t)h * total + q_row0 : ((size_t)b * Hq + h) * S_q) + i] =
                    lt == 0.0f ? -INFINITY : (mu + __builtin_amdgcn_logf(lt)) * kLn2;
        }
    }
}

template <int D, int NW, bool BLK>
hipError_t launch(const PrefillArgs &a, float *bmax, int block_k, hipStream_t stream) {
    const int BG = a.B * a.Hkv;
    const int NB = (a.S + kTile - 1) / kTile;
    // Packed: one slot per 32 rows plus one per sequence, for each KV head.
    const long n_wg = a.cu_seqlens != nullptr
                          ? (long)a.Hkv * (((long)a.total + kTile - 1) / kTile + a.B)
                          : (long)BG * NB;
    if (n_wg * NW * 64 > (long)UINT32_MAX) return hipErrorInvalidConfiguration;
    const int rk = block_k / kTile, NKB = (a.S_kv + block_k - 1) / block_k;
    hipLaunchKernelGGL((stream_attn_kernel<D, NW, BLK>), dim3((unsigned)n_wg), dim3(NW * 64), 0,
                       stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.sink,
                       (bf16 *)a.out, a.lse, a.S, a.S_kv, a.Hq, a.Hkv, a.window, BG, NB, bmax, rk,
                       NKB, a.cu_seqlens, a.total);
    return hipGetLastError();
}

template <int D, bool BLK>
hipError_t launch_d(const PrefillArgs &a, float *bmax, int block_k, hipStream_t stream) {
    switch (waves_for_group(a.Hq / a.Hkv)) {
    case 8: return launch<D, 8, BLK>(a, bmax, block_k, stream);
    case 4: return launch<D, 4, BLK>(a, bmax, block_k, stream);
    case 2: return launch<D, 2, BLK>(a, bmax, block_k, stream);
    default: return launch<D, 1, BLK>(a, bmax, block_k, stream);
    }
}

}  // namespace

hipError_t launch_stream_bf16(const PrefillArgs &a, hipStream_t stream) {
    return a.D == 64 ? launch_d<64, false>(a, nullptr, kTile, stream)
                     : launch_d<128, false>(a, nullptr, kTile, stream);
}

hipError_t launch_stream_bf16_block_max(const PrefillArgs &a, float *bmax, int block_k,
                                        hipStream_t stream) {
    return a.D == 64 ? launch_d<64, true>(a, bmax, block_k, stream)
                     : launch_d<128, true>(a, bmax, block_k, stream);
}

}  // namespace swa
