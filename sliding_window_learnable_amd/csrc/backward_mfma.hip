// backward_mfma.hip -- bf16 MFMA kernels of the attention backward (dq and
// dk/dv) for causal sliding-window / global attention with a per-head sink
// (technical-report digest, 前置知识 / 注意力sink偏置 and 混合注意力机制).
// The sink enters only through lse (from the forward) and through the sink
// gradient, which the pre-pass computes; here P_ij = e^{x_ij - lse_i} and
// dS_ij = P_ij (dP_ij - D_i) with D_i = dO_i . O_i.
//
// Layout conventions as in the forward (v_mfma_f32_32x32x16_bf16, A rows fed
// in the permuted order of score_row_key so that accumulator registers
// 8kk..8kk+7 are the B operand of the next product's kk-th K=16 step).
//
// dq: one work-group per (batch, KV head, 32 query rows, set of at most four
//   query heads of the group), one wave per query head; key tiles stream
//   through LDS (K rows, V rows, K^T).  Four-wave work-groups let two of them
//   share a CU, so one loads its rows while the other computes.
//   Per tile: S^T = K Q^T, dP^T = V dO^T (lane = query), P^T, dS^T, and
//   dQ^T += K^T dS^T.
// dk/dv: one work-group per (batch, KV head, NW consecutive 32-key tiles),
//   two waves per key tile: an S wave (S = Q K^T, P, dV^T += dO^T P; K in
//   registers) and a dP wave (dP = dO V^T, dS = P (dP - D) with P handed
//   over through LDS, dK^T += Q^T dS; V in registers).  The work-group walks
//   every query head of the group and every 32-row query tile that sees one
//   of its keys; Q, dO, lse and D of each (head, query tile) are copied
//   from memory straight into LDS three steps ahead, in rows whose 16-byte
//   chunks are swizzled so that both the row reads (A of S and dP) and the
//   transposing reads (A of dK^T and dV^T) are free of bank conflicts.
//   dk/dv sum over the heads inside the wave, so no reduction across waves
//   or work-groups is needed.
// dk/dv ring (D = 128, windows up to 129 keys): one work-group per run of
//   consecutive key tiles, twelve waves = six key-tile slots of an S wave and
//   a dP wave each; the query tiles that see the run are walked once (heads
//   innermost) and each slot takes the run's next key tile when its current
//   one has seen its last query tile, so every Q/dO tile is staged once per
//   run.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kTile = 32;

// Row of the permuted accumulator layout: register r of lane half hl.
__device__ __forceinline__ int perm_row(int r, int hl) { return 16 * (r >> 3) + 8 * hl + (r & 7); }


// =========================================================================== dq

constexpr int kDqSlots = 4;     // key tiles t, t+1, t+2 landed or landing, t+3 in flight

template <int D>
struct DqSmem {
    bf16 k[kDqSlots][kTile][D];     // K rows (swizzled): A of S^T = K Q^T, read transposed for dQ
    bf16 v[kDqSlots][kTile][D];     // V rows (swizzled): A of dP^T = V dO^T
};

// One work-group per (batch, KV head, 32 query rows, head set), one wave per
// query head: head set hs holds heads hs*NW .. hs*NW+NW-1 of the group (HS
// sets).  Work-groups run KV head fastest (one XCD per KV head), then head
// set, then query block (longest first), then sequence.  Before the key loop a wave also computes, for its
// rows, D_i = dO_i . O_i and lse_i log2(e) (written to the workspace for
// the dk/dv kernel) and the row tile's sink-gradient partial.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ out, const bf16 *__restrict__ dout, const float *__restrict__ lse,
    const float *__restrict__ sink, float *__restrict__ dsum, float *__restrict__ l2g,
    float *__restrict__ part, bf16 *__restrict__ dq, int S, int Hq, int Hkv, int W, int BG, int NB,
    int HS) {
    __shared__ __align__(16) DqSmem<D> sm;
    lds_poison_all(sm);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hl = lane >> 5;
    const int g = blockIdx.x % Hkv;
    const int rest = blockIdx.x / Hkv;
    const int hs = rest % HS;
    const int qb = NB - 1 - (rest / HS) % NB;             // longest query blocks first
    const int b = rest / HS / NB;
    const int G = Hq / Hkv;
    const float c = kLog2e / sqrtf((float)D);
    const float scale = 1.0f / sqrtf((float)D);

    const int i0 = qb * kTile;
    const int p_first = i0, p_last = min(S - 1, i0 + kTile - 1);
    const int T_lo = max(0, p_first - W + 1) / kTile;
    const int T_hi = p_last / kTile;
    const int n_tiles = T_hi - T_lo + 1;

    const uint32_t rs = (uint32_t)Hkv * D * 2;
    const bf16 *kb = k + ((size_t)b * S * Hkv + g) * D;
    const bf16 *vb = v + ((size_t)b * S * Hkv + g) * D;

    const int i = i0 + lq;
    const bool row_ok = i < S;
    const int pq = min(i, S - 1);
    const int kbias = 8 * hl - pq;                         // key - query = 32T + 16(r>>3) + (r&7) + kbias
    auto tile_masked = [&](int T) {
        return kTile * T + kTile - 1 > p_first || kTile * T <= p_last - W;
    };

    // K and V tiles by buffer->LDS copies: 2 * 32 * 2D bytes in 1 KB
    // instructions, IPW per wave (K first, then V), chunks swizzled by row.
    constexpr int CPR = D / 8;                             // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                          // rows per instruction
    constexpr int NI = 2 * kTile / RPI;                    // instructions per tile (K and V)
    constexpr int IPW = NI / NW;
    static_assert(IPW >= 1 && IPW * NW == NI, "DMA split");
    uint32_t dma_off[IPW];
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
        const int row = ((wave * IPW + u) % (NI / 2)) * RPI + lane / CPR;
        dma_off[u] = row * rs + 16 * ((lane % CPR) ^ swz<D>(row));
    }
    auto stage = [&](int T, int sl) {
        const int rows = min(kTile, S - kTile * T);
        const uint32_t bytes = (uint32_t)(rows - 1) * rs + D * 2;
        const size_t off = (size_t)kTile * T * Hkv * D;
        const u32x4 kr = sgpr_rsrc(kb + off, bytes), vr = sgpr_rsrc(vb + off, bytes);
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int ii = wave * IPW + u;                 // uniform
            const bool is_k = ii < NI / 2;
            bf16(*tile)[D] = is_k ? sm.k[sl] : sm.v[sl];
            dma16(is_k ? kr : vr, tile[(ii % (NI / 2)) * RPI], dma_off[u]);
        }
    };
    auto dma_wait = [&](bool newer) {
        if (newer) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    const int arow_r = score_row_key(lq), arow_s = swz<D>(arow_r);
    const int tr_j = lane & 15, tr_d = 16 * ((lane >> 4) & 1) + 4 * (tr_j & 3);

    for (int hh = hs * NW + wave; hh < G; hh += NW * HS) {
        const int h = g * G + hh;
        if (hh != hs * NW + wave) lds_barrier();           // previous head's tiles released

        // K/V tiles 0..2 start copying before the row loads, so the two
        // latencies overlap.
        for (int t = 0; t < 3 && t < n_tiles; ++t) stage(T_lo + t, t);
        bf16x8 qf[D / 16], gf[D / 16];
        float dsum_part = 0.0f;
        const size_t li = ((size_t)b * Hq + h) * S + pq;
        const float lse_i = lse[li];
        {
            const size_t off = (((size_t)b * S + pq) * Hq + h) * D + 8 * hl;
            bf16x8 of[D / 16];
            // The four loads that share a 128-byte line of a row go out
            // back to back.
#pragma unroll
            for (int k4 = 0; k4 < D / 16; k4 += 4) {
#pragma unroll
                for (int ks = k4; ks < k4 + 4; ++ks) qf[ks] = *(const bf16x8 *)(q + off + 16 * ks);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = k4; ks < k4 + 4; ++ks) gf[ks] = *(const bf16x8 *)(dout + off + 16 * ks);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = k4; ks < k4 + 4; ++ks) of[ks] = *(const bf16x8 *)(out + off + 16 * ks);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // D_i = dO_i . O_i by packed bf16 dot products (exact products,
            // fp32 accumulation), two elements per instruction.
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
            {
                const bf16x8 a = gf[ks], o8 = of[ks];
                dsum_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1),
                                                            __builtin_shufflevector(o8, o8, 0, 1), dsum_part, false);
                dsum_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3),
                                                            __builtin_shufflevector(o8, o8, 2, 3), dsum_part, false);
                dsum_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5),
                                                            __builtin_shufflevector(o8, o8, 4, 5), dsum_part, false);
                dsum_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7),
                                                            __builtin_shufflevector(o8, o8, 6, 7), dsum_part, false);
            }
        }
        const float l2 = lse_i * kLog2e;
        const float Di = dsum_part + __shfl_xor(dsum_part, 32);
        {
            // D_i and lse log2(e) for the dk/dv kernel; this row tile's
            // partial of the sink gradient, sum_i e^{s_h - lse_i} D_i.
            if (row_ok && hl == 0) {
                dsum[li] = Di;
                l2g[li] = l2;
            }
            const float sh = sink[h];
            float term = (row_ok && hl == 0 && sh != -INFINITY) ? expf(sh - lse_i) * Di : 0.0f;
            for (int m = 1; m < 64; m <<= 1) term += __shfl_xor(term, m);
            if (lane == 0) part[((size_t)b * Hq + h) * NB + qb] = term;
        }
        f32x16 acc[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            retire(qf[ks]);
            retire(gf[ks]);
        }

        dma_wait(false);
        lds_barrier();

        for (int t = 0; t < n_tiles; ++t) {
            const int T = T_lo + t, sl = t % kDqSlots;
            const bool copy = t + 3 < n_tiles;
            if (copy) stage(T + 3, (t + 3) % kDqSlots);
            const bf16 *krow = sm.k[sl][arow_r];
            const bf16 *vrow = sm.v[sl][arow_r];
            f32x16 st = zero16(), dpt = zero16();
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const int ch = 8 * ((2 * ks + hl) ^ arow_s);
                st = mfma32(*(const bf16x8 *)(krow + ch), qf[ks], st);
                dpt = mfma32(*(const bf16x8 *)(vrow + ch), gf[ks], dpt);
            }
            if (tile_masked(T)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int dk = kTile * T + 16 * (r >> 3) + (r & 7) + kbias;
                    st[r] = (dk <= 0 && dk > -W) ? st[r] : -INFINITY;
                }
            }
            f32x16 ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(st[r], c, -l2));
                ds[r] = p * (dpt[r] - Di);
            }
            const bf16x8 da = pack8(ds, 0), db = pack8(ds, 1);
            // dQ^T += K^T dS^T: A row m = dim 32dt + m, k = key 16kk + 8hl + 0..7,
            // from the K row tile by transposing reads of 4 keys each.
            const bf16(*kt)[D] = sm.k[sl];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int d = 32 * dt + tr_d, cc = d >> 3, half = (d >> 2) & 1;
                bf16x8 a[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int r1 = 16 * kk + 8 * hl + (tr_j >> 2), r2 = r1 + 4;
                    const bf16x4 lo = lds_read_tr(&kt[r1][8 * (cc ^ swz<D>(r1)) + 4 * half]);
                    const bf16x4 hi = lds_read_tr(&kt[r2][8 * (cc ^ swz<D>(r2)) + 4 * half]);
                    a[kk] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
                acc[dt] = mfma32(a[0], da, acc[dt]);
                acc[dt] = mfma32(a[1], db, acc[dt]);
            }
            dma_wait(copy);
            lds_barrier();                                 // tile t's slot released
        }

        // dq rows through this wave's 32 x D area of the (now idle) K/V
        // slots, stored as whole rows: 16 bytes per lane, CPR lanes a row.
        {
            static_assert(sizeof(sm.k) + sizeof(sm.v) >= (size_t)NW * kTile * D * 2, "staging");
            bf16 (*stg)[D] = reinterpret_cast<bf16 (*)[D]>(reinterpret_cast<char *>(&sm)) +
                             wave * kTile;            // K then V slots, from the start of sm
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                u32x2 w[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bf16x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (bf16)(acc[dt][4 * jj + e] * scale);
                    w[jj] = __builtin_bit_cast(u32x2, x);
                    const int cidx = 4 * dt + jj;                 // 16-byte chunk of dims 8*cidx..
                    *(u32x2 *)&stg[lq][8 * (cidx ^ swz<D>(lq)) + 4 * hl] = w[jj];
                }
                lds_settle(w);
            }
#pragma unroll
            for (int u = 0; u < kTile / RPI; ++u) {
                const int r = RPI * u + lane / CPR, cidx = lane % CPR;
                const bf16x8 y = *(const bf16x8 *)&stg[r][8 * (cidx ^ swz<D>(r))];
                if (i0 + r < S)
                    *(bf16x8 *)(dq + (((size_t)b * S + i0 + r) * Hq + h) * D + 8 * cidx) = y;
            }
        }
    }
}

// ========================================================================= dk/dv

constexpr int kKvSlots = 4;     // staging slots: pairs n, n+1 in use, n+2 landed, n+3 in flight

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <int D, int NW>
struct KvSmem {
    bf16 q[kKvSlots][kTile][D];     // Q rows (swizzled): A of S = Q K^T, read transposed for dK
    bf16 g[kKvSlots][kTile][D];     // dO rows (swizzled): A of dP = dO V^T, transposed for dV
    float l2[kKvSlots][kTile];      // lse * log2(e) (0 past the end, where dO = 0)
    float dd[kKvSlots][kTile];      // D_i
    f16x4 px[2][NW][4][64];         // P of each key tile (fp16), from its S wave to its dP wave
};

template <int V>
struct IntC {
    static constexpr int value = V;
};

// NW key tiles per work-group, two waves per tile: waves 0..NW-1 compute
// S = Q K^T, P and dV^T += dO^T P (K in registers); waves NW..2NW-1 compute
// dP = dO V^T, dS = P (dP - D) with P handed over through LDS in fp16 (so
// that a two-tile work-group fits twice in a CU's LDS), and
// dK^T += Q^T dS (V in registers).  The S waves run one pair ahead: in
// step n they compute P of pair n+1 and dV of pair n while the dP waves
// finish pair n, so each step has one barrier.  Q, lse (S waves) and dO, D
// (dP waves) of pair n+3 are copied straight from memory into LDS slot
// (n+3)%4 during step n; P rotates over two buffers.
template <int D, int NW>
__global__ __launch_bounds__(2 * NW * 64) void bwd_dkdv_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ l2g, const float *__restrict__ dsum,
    bf16 *__restrict__ dk, bf16 *__restrict__ dv, int S, int Hq, int Hkv, int W, int BG) {
    __shared__ __align__(16) KvSmem<D, NW> sm;
    lds_poison_all(sm);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool role_s = wave < NW;                         // S/P/dV wave, else dP/dS/dK
    const int slot = role_s ? wave : wave - NW;
    const int lq = lane & 31, hl = lane >> 5;
    const int bg = blockIdx.x % BG;
    const int kblk = blockIdx.x / BG;                      // earliest keys (most queries) first
    const int b = bg / Hkv, g = bg % Hkv;
    const int G = Hq / Hkv;
    const float c = kLog2e / sqrtf((float)D);
    const float scale = 1.0f / sqrtf((float)D);
    const int nQT = (S + kTile - 1) / kTile;

    const int kt = kblk * NW + slot;                       // this wave's key tile
    const int j0 = kt * kTile;
    const bool wave_ok = j0 < S;
    const int qt_lo = kblk * NW;
    const int last_key = min(S - 1, (kblk * NW + NW) * kTile - 1);
    const int qt_hi = (int)min((long)nQT - 1, ((long)last_key + W - 1) / kTile);

    // K (S waves) or V (dP waves) of this tile as B operands: lane = key,
    // dims 16ks + 8hl.  Keys past the end read as zero; their columns are
    // never stored.
    bf16x8 kvf[D / 16];
    {
        const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kTile, S - j0)));
        const uint32_t rs = (uint32_t)Hkv * D * 2;
        const size_t base = (((size_t)b * S + min(j0, S - 1)) * Hkv + g) * D;
        const rsrc_t r = make_rsrc((role_s ? k : v) + base, (uint32_t)rows * rs);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            kvf[ks] = buf_load16(r, lq * rs + 2 * (16 * ks + 8 * hl), 0);
    }
    f32x16 acc[D / 32];                                    // dV^T (S waves) or dK^T
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();

    // Pairs n = (head n / NQ, query tile qt_lo + n % NQ), walked with counters.
    const int NQ = qt_hi - qt_lo + 1, N = G * NQ;
    // Do this tile's keys see any row of query tile qt?  (uniform)
    auto active = [&](int qt) { return wave_ok && qt >= kt && (qt - kt) * kTile < W + kTile - 1; };
    // x = A(pair in buffer bi) . kvf^T: S (S waves) or dP (dP waves), lane = key.
    const int arow_r = score_row_key(lq), arow_s = swz<D>(arow_r);
    auto scores = [&](int bi) {
        const bf16 *arow = role_s ? sm.q[bi][arow_r] : sm.g[bi][arow_r];
        f32x16 x = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            x = mfma32(*(const bf16x8 *)(arow + 8 * ((2 * ks + hl) ^ arow_s)), kvf[ks], x);
        return x;
    };
    // P of a pair with query tile qt (S waves): masked, exponentiated, written to px[pb].
    auto softmax = [&](f32x16 &x, int qt, int pbuf, int bi) {
        const int r0 = qt * kTile;
        // rows i = r0 + perm_row(r, hl), key j = j0 + lq: visible iff j <= i < j + W
        const bool masked = qt == kt || (qt * kTile + kTile - 1) - W >= j0;
        f16x4 *px = sm.px[pbuf][slot][0] + lane;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = 16 * (u >> 1) + 8 * hl + 4 * (u & 1);
            const f32x4 l2v = *(const f32x4 *)&sm.l2[bi][row];
            f16x4 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * u + e;
                float y = x[r];
                if (masked) {
                    const int dij = (r0 + perm_row(r, hl)) - (j0 + lq);
                    y = (dij >= 0 && dij < W) ? y : -INFINITY;
                }
                x[r] = __builtin_amdgcn_exp2f(fmaf(y, c, -l2v[e]));
                pv[e] = (_Float16)x[r];
            }
            px[64 * u] = pv;
        }
    };
    // acc += A^T(buffer bi) . (xa, xb): dV^T (S waves, dO^T) or dK^T (dP waves,
    // Q^T).  A row m = dim 32dt + m, k = query 16kk + 8hl + 0..7, read from the
    // row tile with two transposing reads of 4 queries each.
    const int tr_j = lane & 15, tr_d = 16 * ((lane >> 4) & 1) + 4 * (tr_j & 3);
    auto accumulate = [&](const bf16x8 &xa, const bf16x8 &xb, int bi) {
        const bf16(*t)[D] = role_s ? sm.g[bi] : sm.q[bi];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const int d = 32 * dt + tr_d, c = d >> 3, half = (d >> 2) & 1;
            bf16x8 a[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int r1 = 16 * kk + 8 * hl + (tr_j >> 2), r2 = r1 + 4;
                const bf16x4 lo = lds_read_tr(&t[r1][8 * (c ^ swz<D>(r1)) + 4 * half]);
                const bf16x4 hi = lds_read_tr(&t[r2][8 * (c ^ swz<D>(r2)) + 4 * half]);
                a[kk] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            acc[dt] = mfma32(a[0], xa, acc[dt]);
            acc[dt] = mfma32(a[1], xb, acc[dt]);
        }
    };

    // Staging by DMA: S waves copy Q rows and lse*log2(e), dP waves dO rows
    // and D, of the pairs in order; IPW instructions of 1 KB per wave and
    // tile (wave 0 of each role also copies the 128-byte row vector).
    constexpr int CPR = D / 8;                             // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                          // rows per DMA instruction
    constexpr int IPW = kTile / RPI / NW;                  // instructions per wave and tile
    static_assert(IPW >= 1 && IPW * NW * RPI == kTile, "DMA split");
    const uint32_t qrow_bytes = (uint32_t)Hq * D * 2;
    const bf16 *tsrc = role_s ? q : dout;
    const float *vsrc = role_s ? l2g : dsum;
    uint32_t dma_off[IPW];                                 // row * row_bytes + swizzled chunk
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
        const int row = (slot * IPW + u) * RPI + lane / CPR;
        dma_off[u] = row * qrow_bytes + 16 * ((lane % CPR) ^ swz<D>(row));
    }
    int ld_h = g * G, ld_t = 0;                            // next pair to copy
    auto stage = [&](int sl) {
        const int r0 = (qt_lo + ld_t) * kTile;
        const int rows = min(kTile, S - r0);
        const size_t base = (((size_t)b * S + r0) * Hq + ld_h) * D;
        const u32x4 r = sgpr_rsrc(tsrc + base, (uint32_t)(rows - 1) * qrow_bytes + D * 2);
        bf16(*tile)[D] = role_s ? sm.q[sl] : sm.g[sl];
#pragma unroll
        for (int u = 0; u < IPW; ++u) dma16(r, tile[(slot * IPW + u) * RPI], dma_off[u]);
        if (slot == 0) {
            const u32x4 rv = sgpr_rsrc(vsrc + ((size_t)b * Hq + ld_h) * S + r0, (uint32_t)rows * 4);
            if (lane < kTile / 4) dma16(rv, role_s ? sm.l2[sl] : sm.dd[sl], 16 * lane);
        }
        if (++ld_t == NQ) {
            ld_t = 0;
            ++ld_h;
        }
    };
    // Wait for this wave's copies except those of the current step (newer).
    auto dma_wait = [&](bool newer) {
        if (!newer) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (slot == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW) : "memory");
    };
    for (int n = 0; n < 3 && n < N; ++n) stage(n);       // overlaps the K/V row loads
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) retire(kvf[ks]);
    dma_wait(false);
    lds_barrier();

    bf16x8 pa, pb;                                         // P of pair n (S waves)
    if (role_s && active(qt_lo)) {
        f32x16 x = scores(0);
        softmax(x, qt_lo, 0, 0);
        pa = pack8(x, 0);
        pb = pack8(x, 1);
    }
    lds_barrier();

    // Step n (one barrier each): copy pair n+3 into slot (n+3)%4; S waves:
    // P of pair n+1, dV of pair n; dP waves: dS and dK of pair n; then wait
    // for pair n+2's copy (issued in step n-1) before the barrier.
    int t_cur = 0;                                         // query tile index of pair n
    if (role_s) {
        for (int n = 0; n < N; ++n) {
            const int bi = n % kKvSlots, bn = (n + 1) % kKvSlots;
            const int t_next = t_cur + 1 == NQ ? 0 : t_cur + 1;
            const int qt = qt_lo + t_cur, qn = qt_lo + t_next;
            const bool copy = n + 3 < N;
            if (copy) stage((n + 3) % kKvSlots);
            bf16x8 na, nb;
            const bool next = n + 1 < N && active(qn);
            if (next) {
                f32x16 x = scores(bn);
                softmax(x, qn, (n + 1) & 1, bn);
                na = pack8(x, 0);
                nb = pack8(x, 1);
            }
            if (active(qt)) accumulate(pa, pb, bi);
            if (next) {
                pa = na;
                pb = nb;
            }
            dma_wait(copy);
            lds_barrier();                                 // step n done: slot n%4, px[n&1] free
            t_cur = t_next;
        }
    } else {
        for (int n = 0; n < N; ++n) {
            const int bi = n % kKvSlots;
            const int qt = qt_lo + t_cur;
            const bool copy = n + 3 < N;
            if (copy) stage((n + 3) % kKvSlots);
            if (active(qt)) {
                f32x16 x = scores(bi);
                const f16x4 *px = sm.px[n & 1][slot][0] + lane;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int row = 16 * (u >> 1) + 8 * hl + 4 * (u & 1);
                    const f32x4 ddv = *(const f32x4 *)&sm.dd[bi][row];
                    const f16x4 pv = px[64 * u];
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[4 * u + e] = pv[e] * (x[4 * u + e] - ddv[e]);
                }
                accumulate(pack8(x, 0), pack8(x, 1), bi);
            }
            dma_wait(copy);
            lds_barrier();                                 // step n done
            t_cur = t_cur + 1 == NQ ? 0 : t_cur + 1;
        }
    }

    // dk / dv rows through this wave's 32 x D area of the (now idle) Q/dO
    // slots, stored as whole rows: 16 bytes per lane, CPR lanes a row.
    if (wave_ok) {
        bf16 *dst = role_s ? dv : dk;
        const float f = role_s ? 1.0f : scale;
        static_assert(sizeof(sm.q) + sizeof(sm.g) >= (size_t)2 * NW * kTile * D * 2, "staging");
        bf16 (*stg)[D] = reinterpret_cast<bf16 (*)[D]>(reinterpret_cast<char *>(&sm)) +
                         wave * kTile;                // Q then dO slots, from the start of sm
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            u32x2 w[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 xo;
#pragma unroll
                for (int e = 0; e < 4; ++e) xo[e] = (bf16)(acc[dt][4 * jj + e] * f);
                w[jj] = __builtin_bit_cast(u32x2, xo);
                const int cidx = 4 * dt + jj;
                *(u32x2 *)&stg[lq][8 * (cidx ^ swz<D>(lq)) + 4 * hl] = w[jj];
            }
            lds_settle(w);
        }
        constexpr int CPR2 = D / 8, RPI2 = 64 / CPR2;
#pragma unroll
        for (int u = 0; u < kTile / RPI2; ++u) {
            const int r = RPI2 * u + lane / CPR2, cidx = lane % CPR2;
            const bf16x8 y = *(const bf16x8 *)&stg[r][8 * (cidx ^ swz<D>(r))];
            if (j0 + r < S)
                *(bf16x8 *)(dst + (((size_t)b * S + j0 + r) * Hkv + g) * D + 8 * cidx) = y;
        }
    }
}

// ==================================================================== dk/dv ring
// For windows up to 129 keys a query tile sees at most five key tiles, so a
// work-group can own a run of consecutive key tiles and walk the query tiles
// that see them once, in order, heads innermost.  Key tile j of the run lives
// in slot (j - k0) mod 6, with two waves per slot as in bwd_dkdv_kernel (S
// wave: S = Q K^T, P, dV^T += dO^T P; dP wave: dP = dO V^T, dS, dK^T += Q^T dS).
// A slot's tile is live for the query tiles that see it (at most five) and
// idle for at least one more; in the first step of that idle span its two
// waves write dv / dk out as whole rows through an LDS area, copy the slot's
// next key tile (K for the S wave, V for the dP wave) into the same area and
// take it into registers.  Each Q / dO tile is then copied once per
// work-group (plus a tail of nvis - 1 query tiles per run) rather than once
// for every two key tiles.
constexpr int kRingSlots = 6;

template <int D>
struct KvRingSmem {
    bf16 q[kKvSlots][kTile][D];     // Q rows (swizzled), as in KvSmem
    bf16 g[kKvSlots][kTile][D];     // dO rows (swizzled)
    float l2[kKvSlots][kTile];      // lse * log2(e)
    float dd[kKvSlots][kTile];      // D_i
    f16x4 px[2][kRingSlots][4][64]; // P of each slot's key tile, S wave -> dP wave
    bf16 stg[2][kTile][D];          // retiring slot: dv (S wave) / dk rows out, then its next K / V in
};

template <int D>
__global__ __launch_bounds__(2 * kRingSlots * 64) void bwd_dkdv_ring_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ l2g, const float *__restrict__ dsum,
    bf16 *__restrict__ dk, bf16 *__restrict__ dv, int S, int Hq, int Hkv, int W, int BG, int run) {
    constexpr int NS = kRingSlots;
    constexpr int CPR = D / 8;                             // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                          // rows per copy instruction
    constexpr int TI = kTile / RPI;                        // copy instructions per tile
    constexpr int CW = 4;                                  // copying waves per role
    constexpr int IPW = TI / CW;                           // ... instructions each
    static_assert(IPW >= 1 && IPW * CW == TI, "copy split");
    __shared__ __align__(16) KvRingSmem<D> sm;
    lds_poison_all(sm);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool role_s = wave < NS;                         // S/P/dV wave, else dP/dS/dK
    const int slot = role_s ? wave : wave - NS;
    const bool copier = slot < CW;
    const int lq = lane & 31, hl = lane >> 5;
    const int bg = blockIdx.x % BG;
    const int b = bg / Hkv, g = bg % Hkv;
    const int G = Hq / Hkv;
    const float c = kLog2e / sqrtf((float)D);
    const float scale = 1.0f / sqrtf((float)D);
    const int nQT = (S + kTile - 1) / kTile;
    const int k0 = (blockIdx.x / BG) * run;                // this run's key tiles: [k0, k_end)
    const int k_end = min(nQT, k0 + run);
    const int nvis = (W + kTile - 2) / kTile + 1;          // query tiles that see one key tile
    const int t_end = min(nQT - 1, k_end - 1 + nvis - 1);  // last query tile of the walk
    const uint32_t rs = (uint32_t)Hkv * D * 2;
    const uint32_t qrow_bytes = (uint32_t)Hq * D * 2;

    int kt = k0 + slot;                                    // this slot's key tile (k_end: none)
    auto active = [&](int qt) __attribute__((always_inline)) {
        return kt < k_end && qt >= kt && (qt - kt) * kTile < W + kTile - 1;
    };

    // The first key tile of the slot as B operands (lane = key, dims 16ks + 8hl).
    bf16x8 kvf[D / 16];
    {
        const int j0 = kt * kTile;
        const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kTile, S - j0)));
        const size_t base = (((size_t)b * S + min(j0, S - 1)) * Hkv + g) * D;
        const rsrc_t r = make_rsrc((role_s ? k : v) + base, (uint32_t)rows * rs);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            kvf[ks] = buf_load16(r, lq * rs + 2 * (16 * ks + 8 * hl), 0);
    }
    f32x16 acc[D / 32];                                    // dV^T (S waves) or dK^T
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();

    const int N = (t_end - k0 + 1) * G;                    // pairs (query tile, head), heads inner
    // Operand addresses.  With 256-byte rows, chunk (2ks + hl) ^ s of a row
    // (s = swz(row)) sits at byte 16((hl ^ s) & 1) + 32(ks ^ (s >> 1)): one
    // per-lane base XOR 32ks.  Transposing reads of rows r1 = 16kk + 8hl +
    // j4 and r1 + 4 (j4 = tr_j / 4), dims 32dt + tr_d: bytes 4096kk + base_rr
    // XOR 64dt, the row's swizzle putting j4 in bits 6-7.  The bases are
    // made opaque where they are used, so that the compiler recomputes the
    // few XORs instead of keeping every read address live in the loop.
    static_assert(D == 128, "ring kernel address scheme: 256-byte rows");
    const int arow_r = score_row_key(lq), arow_s = swz<D>(arow_r);
    const uint32_t sc_off = 256 * arow_r + 16 * ((hl ^ arow_s) & 1) + 32 * (arow_s >> 1);
    const uint32_t role_a = lds_addr(role_s ? &sm.q[0][0][0] : &sm.g[0][0][0]);  // A of S / dP
    const uint32_t role_t = lds_addr(role_s ? &sm.g[0][0][0] : &sm.q[0][0][0]);  // transposed A
    constexpr uint32_t kTileB = kTile * D * 2;
    auto scores = [&](int bi) __attribute__((always_inline)) {
        uint32_t base = role_a + sc_off;
        asm volatile("" : "+v"(base));
        base += bi * kTileB;
        f32x16 x = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) x = mfma32(lds_read16_at(base ^ (32u * ks)), kvf[ks], x);
        // Operand reads two products ahead (few registers at three waves a SIMD).
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 5);
#pragma unroll
        for (int ks = 0; ks < D / 16 - 2; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 5);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 5);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 5);
        return x;
    };
    auto softmax = [&](f32x16 &x, int qt, int pbuf, int bi) __attribute__((always_inline)) {
        const int r0 = qt * kTile, j0 = kt * kTile;
        const bool masked = qt == kt || (qt * kTile + kTile - 1) - W >= j0;
        f16x4 *px = sm.px[pbuf][slot][0] + lane;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = 16 * (u >> 1) + 8 * hl + 4 * (u & 1);
            const f32x4 l2v = *(const f32x4 *)&sm.l2[bi][row];
            f16x4 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * u + e;
                float y = x[r];
                if (masked) {
                    const int dij = (r0 + perm_row(r, hl)) - (j0 + lq);
                    y = (dij >= 0 && dij < W) ? y : -INFINITY;
                }
                x[r] = __builtin_amdgcn_exp2f(fmaf(y, c, -l2v[e]));
                pv[e] = (_Float16)x[r];
            }
            px[64 * u] = pv;
        }
    };
    const int tr_j = lane & 15, tr_d = 16 * ((lane >> 4) & 1) + 4 * (tr_j & 3);
    uint32_t tr_off[2];
    {
        const int j4 = tr_j >> 2, c0 = tr_d >> 3, half = (tr_d >> 2) & 1;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int r = 8 * hl + j4 + 4 * rr;                 // kk = 0
            tr_off[rr] = 256 * r + 16 * (c0 ^ (swz<D>(r) & 3)) + 8 * half + 64 * (swz<D>(r) >> 2);
        }
    }
    auto accumulate = [&](const bf16x8 &xa, const bf16x8 &xb, int bi) __attribute__((always_inline)) {
        uint32_t b0 = role_t + tr_off[0], b1 = role_t + tr_off[1];
        asm volatile("" : "+v"(b0), "+v"(b1));
        b0 += bi * kTileB;
        b1 += bi * kTileB;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const uint32_t a0 = b0 ^ (64u * dt), a1 = b1 ^ (64u * dt);
            bf16x8 a[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x4 lo = lds_read_tr_at(a0 + 4096u * kk);
                const bf16x4 hi = lds_read_tr_at(a1 + 4096u * kk);
                a[kk] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            acc[dt] = mfma32(a[0], xa, acc[dt]);
            acc[dt] = mfma32(a[1], xb, acc[dt]);
        }
        // Transposing reads (two per operand) one product ahead.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 6);
#pragma unroll
        for (int i = 0; i < D / 16 - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 6);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 6);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 6);
    };

    // Q / dO rows of the pairs in order (S waves Q and lse*log2(e), dP waves
    // dO and D); waves of slots 0..CW-1 copy IPW instructions each, slot 0
    // also the 128-byte row vector.
    const bf16 *tsrc = role_s ? q : dout;
    const float *vsrc = role_s ? l2g : dsum;
    uint32_t dma_off[IPW];
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
        const int row = (slot * IPW + u) * RPI + lane / CPR;
        dma_off[u] = row * qrow_bytes + 16 * ((lane % CPR) ^ swz<D>(row));
    }
    int ld_t = k0, ld_h = 0;                               // next pair to copy
    auto stage = [&](int sl) __attribute__((always_inline)) {
        if (copier) {
            const int r0 = ld_t * kTile;
            const int rows = min(kTile, S - r0);
            const int hq = g * G + ld_h;
            const size_t base = (((size_t)b * S + r0) * Hq + hq) * D;
            const u32x4 r = sgpr_rsrc(tsrc + base, (uint32_t)(rows - 1) * qrow_bytes + D * 2);
            bf16(*tile)[D] = role_s ? sm.q[sl] : sm.g[sl];
#pragma unroll
            for (int u = 0; u < IPW; ++u) dma16(r, tile[(slot * IPW + u) * RPI], dma_off[u]);
            if (slot == 0) {
                const u32x4 rv = sgpr_rsrc(vsrc + ((size_t)b * Hq + hq) * S + r0, (uint32_t)rows * 4);
                if (lane < kTile / 4) dma16(rv, role_s ? sm.l2[sl] : sm.dd[sl], 16 * lane);
            }
        }
        if (++ld_h == G) {
            ld_h = 0;
            ++ld_t;
        }
    };
    // Wait for this wave's copies except those of the current step (newer).
    auto dma_wait = [&](bool newer) __attribute__((always_inline)) {
        if (!newer || !copier) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (slot == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW) : "memory");
    };

    // Retire the slot's key tile: dv (S wave) or dk rows through the LDS
    // area st, stored as whole rows; then, with more = true and a next tile
    // in the run, copy that tile (K or V) into the same area.  Returns with
    // the stores complete (their data registers held until then) and the
    // copy in flight.  In the walk one slot retires per query tile, through
    // the role's area of sm.stg.
    bf16(*stg)[D] = sm.stg[role_s ? 0 : 1];
    auto retire_tile = [&](bf16(*st)[D], bool more) __attribute__((always_inline)) {
        // Lane-derived addresses computed here, not kept live through the walk.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lq = ln & 31, hl = ln >> 5;
        const int lane = ln;
        const int j0 = kt * kTile;
        const float f = role_s ? 1.0f : scale;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            u32x2 w[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 xo;
#pragma unroll
                for (int e = 0; e < 4; ++e) xo[e] = (bf16)(acc[dt][4 * jj + e] * f);
                w[jj] = __builtin_bit_cast(u32x2, xo);
                const int cidx = 4 * dt + jj;
                *(u32x2 *)&st[lq][8 * (cidx ^ swz<D>(lq)) + 4 * hl] = w[jj];
            }
            lds_settle(w);
        }
        // Rows out in two halves, each held until its stores are complete
        // (fewer registers live at once); the next tile's copy after them.
        const int rows = __builtin_amdgcn_readfirstlane(min(kTile, S - j0));
        const rsrc_t rd = make_rsrc((role_s ? dv : dk) + (((size_t)b * S + j0) * Hkv + g) * D,
                                    (uint32_t)rows * rs);
        kt += NS;
        const bool copy_next = more && kt < k_end;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            bf16x8 y[TI / 2];
#pragma unroll
            for (int u = 0; u < TI / 2; ++u) {
                const int r = RPI * (TI / 2 * hf + u) + lane / CPR, cidx = lane % CPR;
                y[u] = *(const bf16x8 *)&st[r][8 * (cidx ^ swz<D>(r))];
            }
#pragma unroll
            for (int u = 0; u < TI / 2; ++u)
                buf_store16(y[u], rd, (uint32_t)(RPI * (TI / 2 * hf + u) + lane / CPR) * rs +
                                          16 * (lane % CPR), 0);
            if (hf == 1 && copy_next) {
                // The read-back is complete (the stores consumed it).
                const int j1 = kt * kTile;
                const int rows1 = __builtin_amdgcn_readfirstlane(min(kTile, S - j1));
                const u32x4 r = sgpr_rsrc((role_s ? k : v) + (((size_t)b * S + j1) * Hkv + g) * D,
                                          (uint32_t)(rows1 - 1) * rs + D * 2);
                const uint32_t st_lds = __builtin_amdgcn_readfirstlane(lds_addr(&st[0][0]));
#pragma unroll
                for (int u = 0; u < TI; ++u) {
                    const int row = RPI * u + lane / CPR;
                    dma16_at(r, st_lds + 1024u * u, row * rs + 16 * ((lane % CPR) ^ swz<D>(row)), 0);
                }
                hold_until_done<TI>(y);
            } else {
                hold_until_done<0>(y);
            }
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();
    };
    // The slot's key tile from stg into the B-operand registers (after its copy landed).
    auto take_tile = [&]() __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lq = ln & 31, hl = ln >> 5;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            kvf[ks] = *(const bf16x8 *)&stg[lq][8 * ((2 * ks + hl) ^ swz<D>(lq))];
    };

    for (int n = 0; n < 3 && n < N; ++n) stage(n);       // overlaps the K/V row loads
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) retire(kvf[ks]);
    dma_wait(false);
    lds_barrier();

    bf16x8 pa, pb;                                         // P of pair n (S waves)
    if (role_s && active(k0)) {
        f32x16 x = scores(0);
        softmax(x, k0, 0, 0);
        pa = pack8(x, 0);
        pb = pack8(x, 1);
    }
    lds_barrier();

    // Step n: the slot retires its tile if pair n is the first after the
    // tile's last (the next tile is taken at once when pair n+1, the S wave's
    // look-ahead, already needs it, else after this step's wait); copy pair
    // n+3 into slot (n+3)%4; S waves: dV of pair n, P of pair n+1; dP waves:
    // dS and dK of pair n; wait for pair n+2's copy.
    auto maybe_retire = [&](int t_cur, int h_cur, int t_next, int n) __attribute__((always_inline)) {
        bool take_late = false;
        if (h_cur == 0 && kt < k_end && t_cur == kt + nvis) {
            retire_tile(stg, true);
            if (kt < k_end) {
                if (role_s && n + 1 < N && active(t_next)) {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    take_tile();
                } else {
                    take_late = true;
                }
            }
        }
        return take_late;
    };
    int t_cur = k0, h_cur = 0;                             // pair n
    if (role_s) {
        for (int n = 0; n < N; ++n) {
            const int bi = n % kKvSlots, bn = (n + 1) % kKvSlots;
            const int t_next = h_cur + 1 == G ? t_cur + 1 : t_cur;
            const bool take_late = maybe_retire(t_cur, h_cur, t_next, n);
            const bool copy = n + 3 < N;
            if (copy) stage((n + 3) % kKvSlots);
            // dV of pair n first, then P of pair n+1, kept apart so that the
            // two products' operand reads are never live together.
            if (active(t_cur)) accumulate(pa, pb, bi);
            __builtin_amdgcn_sched_barrier(0);
            if (n + 1 < N && active(t_next)) {
                f32x16 x = scores(bn);
                softmax(x, t_next, (n + 1) & 1, bn);
                pa = pack8(x, 0);
                pb = pack8(x, 1);
            }
            dma_wait(copy);                                // also the retirement's tile copy
            if (take_late) take_tile();
            lds_barrier();                                 // step n done
            t_cur = t_next;
            h_cur = h_cur + 1 == G ? 0 : h_cur + 1;
        }
    } else {
        for (int n = 0; n < N; ++n) {
            const int bi = n % kKvSlots;
            const int t_next = h_cur + 1 == G ? t_cur + 1 : t_cur;
            const bool take_late = maybe_retire(t_cur, h_cur, t_next, n);
            const bool copy = n + 3 < N;
            if (copy) stage((n + 3) % kKvSlots);
            if (active(t_cur)) {
                f32x16 x = scores(bi);
                const f16x4 *px = sm.px[n & 1][slot][0] + lane;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int row = 16 * (u >> 1) + 8 * hl + 4 * (u & 1);
                    const f32x4 ddv = *(const f32x4 *)&sm.dd[bi][row];
                    const f16x4 pv = px[64 * u];
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[4 * u + e] = pv[e] * (x[4 * u + e] - ddv[e]);
                }
                accumulate(pack8(x, 0), pack8(x, 1), bi);
            }
            dma_wait(copy);
            if (take_late) take_tile();
            lds_barrier();                                 // step n done
            t_cur = t_next;
            h_cur = h_cur + 1 == G ? 0 : h_cur + 1;
        }
    }
    // Tiles still live at the end of the walk (up to one per slot) retire
    // together, each wave through its own 32 x D area of the now idle LDS.
    lds_barrier();
    static_assert(sizeof(sm) >= (size_t)2 * NS * kTile * D * 2, "final staging");
    if (kt < k_end)
        retire_tile(reinterpret_cast<bf16(*)[D]>(reinterpret_cast<char *>(&sm)) + wave * kTile, false);
}

template <int D, int NW>
hipError_t launch_dq(const BackwardArgs &a, hipStream_t stream) {
    const int BG = a.B * a.Hkv;
    const int NB = (a.S + kTile - 1) / kTile;
    const int HS = (a.Hq / a.Hkv) / NW;                    // head sets per group
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW>), dim3((unsigned)((long)BG * NB * HS)), dim3(NW * 64), 0,
                       stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                       (const bf16 *)a.out, (const bf16 *)a.dout, a.lse, a.sink, a.ws_dsum, a.ws_l2,
                       a.ws_part, (bf16 *)a.dq, a.S, a.Hq, a.Hkv, a.window, BG, NB, HS);
    return hipGetLastError();
}

// Key tiles per dk/dv work-group (two waves each).  A work-group walks the
// query tiles that see any of its keys, so narrow windows read each Q/dO
// tile (NW + nvis - 1) / NW times, nvis being the query tiles one key tile
// sees; two key tiles read more of them than four, but two such work-groups
// share a CU and hide each other's copy latency.  Measured at S = 32768:
// two tiles win up to window 256 (1.124 vs 1.201 ms at 128), tie at 512,
// and lose from 1024 on (5.01 vs 4.77 ms) and for the global layer.
template <int D, int NW>
hipError_t launch_dkdv_nw(const BackwardArgs &a, hipStream_t stream) {
    const int BG = a.B * a.Hkv;
    const int nKT = (a.S + kTile - 1) / kTile;
    const int nblk = (nKT + NW - 1) / NW;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW>), dim3((unsigned)((long)BG * nblk)), dim3(2 * NW * 64),
                       0, stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                       (const bf16 *)a.dout, a.ws_l2, a.ws_dsum, (bf16 *)a.dk, (bf16 *)a.dv, a.S,
                       a.Hq, a.Hkv, a.window, BG);
    return hipGetLastError();
}

// Key tiles per ring work-group: enough work-groups to give every CU one,
// at least one tile per slot.
hipError_t launch_dkdv_ring(const BackwardArgs &a, hipStream_t stream) {
    constexpr int D = 128;
    const int BG = a.B * a.Hkv;
    const int nKT = (a.S + kTile - 1) / kTile;
    const long want = 256;
    const int run = (int)max((long)kRingSlots, ((long)nKT * BG + want - 1) / want);
    const int nrun = (nKT + run - 1) / run;
    hipLaunchKernelGGL((bwd_dkdv_ring_kernel<D>), dim3((unsigned)((long)BG * nrun)),
                       dim3(2 * kRingSlots * 64), 0, stream, (const bf16 *)a.q, (const bf16 *)a.k,
                       (const bf16 *)a.v, (const bf16 *)a.dout, a.ws_l2, a.ws_dsum, (bf16 *)a.dk,
                       (bf16 *)a.dv, a.S, a.Hq, a.Hkv, a.window, BG, run);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv(const BackwardArgs &a, hipStream_t stream) {
    if constexpr (D == 128)
        if (a.window <= 129) return launch_dkdv_ring(a, stream);
    return a.window <= 256 ? launch_dkdv_nw<D, 2>(a, stream) : launch_dkdv_nw<D, 4>(a, stream);
}

template <int D>
hipError_t launch_d(const BackwardArgs &a, hipStream_t stream) {
    hipError_t e;
    switch (waves_for_group(a.Hq / a.Hkv)) {
    case 8:
    case 4: e = launch_dq<D, 4>(a, stream); break;
    case 2: e = launch_dq<D, 2>(a, stream); break;
    default: e = launch_dq<D, 1>(a, stream); break;
    }
    if (e != hipSuccess) return e;
    e = launch_backward_dsink(a, stream);
    if (e != hipSuccess) return e;
    return launch_dkdv<D>(a, stream);
}

}  // namespace

// dq (with D_i, lse log2(e) and the sink-gradient partials), the sink
// gradient, then dk/dv (which reads D_i and lse log2(e)).
hipError_t launch_backward_bf16(const BackwardArgs &a, hipStream_t stream) {
    return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace swa
