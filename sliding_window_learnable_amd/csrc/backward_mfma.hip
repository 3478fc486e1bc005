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
// dq: one work-group per (batch, KV head, 32 query rows), one wave per query
//   head of the group; key tiles stream through LDS (K rows, V rows, K^T).
//   Per tile: S^T = K Q^T, dP^T = V dO^T (lane = query), P^T, dS^T, and
//   dQ^T += K^T dS^T.
// dk/dv: one work-group per (batch, KV head, NW consecutive 32-key tiles),
//   one wave per key tile; K and V of the wave's tile stay in registers as
//   the B operands.  The work-group walks every query head of the group and
//   every 32-row query tile that sees one of its keys, staging Q, dO (rows
//   and transposed), lse and D once for all its waves.  Per (head, query
//   tile) a wave computes S = Q K^T and dP = dO V^T (lane = key), P, dS, and
//   dV^T += dO^T P, dK^T += Q^T dS; dk/dv sum over the heads inside the wave,
//   so no reduction across waves or work-groups is needed.
#include "attn_device.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kTile = 32;

// Row of the permuted accumulator layout: register r of lane half hl.
__device__ __forceinline__ int perm_row(int r, int hl) { return 16 * (r >> 3) + 8 * hl + (r & 7); }

// 4 rows x 8 dims quad written transposed: dst[8ch + e][col..col+3].
template <int LD>
__device__ __forceinline__ void store_transposed(bf16 (*dst)[LD], const bf16x8 (&quad)[4], int ch,
                                                 int col) {
    u32x2 w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bf16x4 x;
        x[0] = quad[0][e];
        x[1] = quad[1][e];
        x[2] = quad[2][e];
        x[3] = quad[3][e];
        w[e] = __builtin_bit_cast(u32x2, x);
        *(u32x2 *)&dst[8 * ch + e][col] = w[e];
    }
    lds_settle(w);
}

// =========================================================================== dq

template <int D>
struct DqSmem {
    bf16 k[2][kTile][D + 8];
    bf16 v[2][kTile][D + 8];
    bf16 kt[2][D][kTile + 8];
};

// One 32-key tile: K and V as 4-row x 8-dim quads (rows past the end read
// zeros); K rows, V rows and K^T are written to a slot.
template <int D, int NT>
struct DqLoader {
    static constexpr int CH = D / 8;
    static constexpr int QPT = (2 * 8 * CH + NT - 1) / NT;   // K and V quads per thread
    bf16x8 quad[QPT][4];

    __device__ __forceinline__ void load(const bf16 *kb, const bf16 *vb, size_t row_elems,
                                         uint32_t rs, int S, int T, int tid) {
        const int rows = min(kTile, S - kTile * T);
        const uint32_t bytes = rows > 0 ? (uint32_t)rows * rs : 0u;
        const rsrc_t kr = make_rsrc(kb + (size_t)kTile * T * row_elems, bytes);
        const rsrc_t vr = make_rsrc(vb + (size_t)kTile * T * row_elems, bytes);
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
            const int item = tid + i * NT;
            if (item < 2 * 8 * CH) {                        // wave-uniform (multiples of 64)
                const int it = item % (8 * CH), kq = it & 7, ch = it >> 3;
                // K or V: the same for the whole wave (64-aligned item ranges),
                // stated so that the descriptor stays scalar.
                const bool is_k = __builtin_amdgcn_readfirstlane(item / (8 * CH)) == 0;
                const rsrc_t r = is_k ? kr : vr;
#pragma unroll
                for (int j = 0; j < 4; ++j) quad[i][j] = buf_load16(r, (4 * kq + j) * rs + 16 * ch, 0);
            }
        }
    }

    __device__ __forceinline__ void store(DqSmem<D> &sm, int slot, int tid) const {
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
            const int item = tid + i * NT;
            if (item < 2 * 8 * CH) {
                const bool is_k = __builtin_amdgcn_readfirstlane(item / (8 * CH)) == 0;
                const int it = item % (8 * CH), kq = it & 7, ch = it >> 3;
                bf16(*rows)[D + 8] = is_k ? sm.k[slot] : sm.v[slot];
#pragma unroll
                for (int j = 0; j < 4; ++j) *(bf16x8 *)&rows[4 * kq + j][8 * ch] = quad[i][j];
                lds_settle(quad[i]);
                if (is_k) store_transposed(sm.kt[slot], quad[i], ch, 4 * kq);
            }
        }
    }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ dsum,
    bf16 *__restrict__ dq, int S, int Hq, int Hkv, int W, int BG, int NB) {
    constexpr int NT = NW * 64;
    __shared__ __align__(16) DqSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hl = lane >> 5;
    const int bg = blockIdx.x % BG;
    const int qb = NB - 1 - blockIdx.x / BG;              // longest query blocks first
    const int b = bg / Hkv, g = bg % Hkv;
    const int G = Hq / Hkv;
    const float c = kLog2e / sqrtf((float)D);
    const float scale = 1.0f / sqrtf((float)D);

    const int i0 = qb * kTile;
    const int p_first = i0, p_last = min(S - 1, i0 + kTile - 1);
    const int T_lo = max(0, p_first - W + 1) / kTile;
    const int T_hi = p_last / kTile;
    const int n_tiles = T_hi - T_lo + 1;

    const size_t row_elems = (size_t)Hkv * D;
    const uint32_t rs = (uint32_t)row_elems * 2;
    const bf16 *kb = k + ((size_t)b * S * Hkv + g) * D;
    const bf16 *vb = v + ((size_t)b * S * Hkv + g) * D;

    const int i = i0 + lq;
    const bool row_ok = i < S;
    const int pq = min(i, S - 1);
    const int kbias = 8 * hl - pq;                         // key - query = 32T + 16(r>>3) + (r&7) + kbias
    auto tile_masked = [&](int T) {
        return kTile * T + kTile - 1 > p_first || kTile * T <= p_last - W;
    };

    DqLoader<D, NT> ld;
    for (int hh = wave; hh < G; hh += NW) {
        const int h = g * G + hh;
        if (hh != wave) lds_barrier();
        ld.load(kb, vb, row_elems, rs, S, T_lo, tid);
        ld.store(sm, 0, tid);
        lds_barrier();

        bf16x8 qf[D / 16], gf[D / 16];
        {
            const size_t off = (((size_t)b * S + pq) * Hq + h) * D + 8 * hl;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                qf[ks] = *(const bf16x8 *)(q + off + 16 * ks);
                gf[ks] = *(const bf16x8 *)(dout + off + 16 * ks);
            }
        }
        const size_t li = ((size_t)b * Hq + h) * S + pq;
        const float l2 = lse[li] * kLog2e;
        const float Di = dsum[li];
        f32x16 acc[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();

        for (int t = 0; t < n_tiles; ++t) {
            const int T = T_lo + t, slot = t & 1;
            if (t + 1 < n_tiles) ld.load(kb, vb, row_elems, rs, S, T + 1, tid);
            const bf16 *krow = &sm.k[slot][score_row_key(lq)][8 * hl];
            const bf16 *vrow = &sm.v[slot][score_row_key(lq)][8 * hl];
            f32x16 st = mfma32(*(const bf16x8 *)krow, qf[0], zero16());
            f32x16 dpt = mfma32(*(const bf16x8 *)vrow, gf[0], zero16());
#pragma unroll
            for (int ks = 1; ks < D / 16; ++ks) {
                st = mfma32(*(const bf16x8 *)(krow + 16 * ks), qf[ks], st);
                dpt = mfma32(*(const bf16x8 *)(vrow + 16 * ks), gf[ks], dpt);
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
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                acc[dt] = mfma32(*(const bf16x8 *)&sm.kt[slot][32 * dt + lq][8 * hl], da, acc[dt]);
                acc[dt] = mfma32(*(const bf16x8 *)&sm.kt[slot][32 * dt + lq][16 + 8 * hl], db, acc[dt]);
            }
            if (t + 1 < n_tiles) ld.store(sm, (t + 1) & 1, tid);
            lds_barrier();
        }

        if (row_ok) {
            bf16 *orow = dq + (((size_t)b * S + i) * Hq + h) * D;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bf16x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (bf16)(acc[dt][4 * jj + e] * scale);
                    *(bf16x4 *)(orow + 32 * dt + 8 * jj + 4 * hl) = x;
                }
        }
    }
}

// ========================================================================= dk/dv

template <int D, int NW>
struct KvSmem {
    bf16 kw[NW][kTile][D + 8];  // each wave's K rows: B of S = Q K^T
    bf16 vw[NW][kTile][D + 8];  // each wave's V rows: B of dP = dO V^T
    bf16 q[2][kTile][D + 8];    // Q rows: A of S = Q K^T
    bf16 g[2][kTile][D + 8];    // dO rows: A of dP = dO V^T
    bf16 qt[2][D][kTile + 8];   // Q^T: A of dK^T = Q^T dS
    bf16 gt[2][D][kTile + 8];   // dO^T: A of dV^T = dO^T P
    float l2[2][kTile];         // lse * log2(e); +inf past the end (P = 0)
    float dd[2][kTile];         // D_i
};

// One (head, 32-row query tile) of Q and dO as 4-row x 8-dim quads plus the
// rows' lse and D, loaded into registers, then written to an LDS buffer as
// rows and transposed.
template <int D, int NT>
struct KvStager {
    static constexpr int CH = D / 8;
    static constexpr int QPT = (2 * 8 * CH + NT - 1) / NT;  // Q and dO quads per thread
    bf16x8 quad[QPT][4];
    float l2, dd;

    __device__ __forceinline__ void load(const bf16 *q, const bf16 *dout, const float *lse,
                                         const float *dsum, int b, int h, int r0, int S, int Hq,
                                         int tid) {
        const int rows = min(kTile, S - r0);
        const uint32_t qrow_bytes = (uint32_t)Hq * D * 2;
        const uint32_t bytes = (uint32_t)(rows - 1) * qrow_bytes + D * 2;
        const size_t base = (((size_t)b * S + r0) * Hq + h) * D;
        const rsrc_t qr = make_rsrc(q + base, bytes);
        const rsrc_t gr = make_rsrc(dout + base, bytes);
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int item = tid + u * NT;
            if (item < 2 * 8 * CH) {                        // wave-uniform
                const int it = item % (8 * CH), kq = it & 7, ch = it >> 3;
                // Q or dO: the same for the whole wave (64-aligned item ranges),
                // stated so that the descriptor stays scalar.
                const bool is_q = __builtin_amdgcn_readfirstlane(item / (8 * CH)) == 0;
                const rsrc_t r = is_q ? qr : gr;
#pragma unroll
                for (int j = 0; j < 4; ++j) quad[u][j] = buf_load16(r, (4 * kq + j) * qrow_bytes + 16 * ch, 0);
            }
        }
        if (tid < kTile) {
            const bool ok = tid < rows;
            const size_t li = ((size_t)b * Hq + h) * S + r0 + (ok ? tid : 0);
            l2 = ok ? lse[li] * kLog2e : INFINITY;
            dd = ok ? dsum[li] : 0.0f;
        }
    }

    template <class Smem>
    __device__ __forceinline__ void store(Smem &sm, int buf, int tid) const {
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int item = tid + u * NT;
            if (item < 2 * 8 * CH) {
                const bool is_q = __builtin_amdgcn_readfirstlane(item / (8 * CH)) == 0;
                const int it = item % (8 * CH), kq = it & 7, ch = it >> 3;
                bf16(*rws)[D + 8] = is_q ? sm.q[buf] : sm.g[buf];
#pragma unroll
                for (int j = 0; j < 4; ++j) *(bf16x8 *)&rws[4 * kq + j][8 * ch] = quad[u][j];
                lds_settle(quad[u]);
                store_transposed(is_q ? sm.qt[buf] : sm.gt[buf], quad[u], ch, 4 * kq);
            }
        }
        if (tid < kTile) {
            sm.l2[buf][tid] = l2;
            sm.dd[buf][tid] = dd;
        }
    }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ dsum,
    bf16 *__restrict__ dk, bf16 *__restrict__ dv, int S, int Hq, int Hkv, int W, int BG) {
    constexpr int NT = NW * 64;
    __shared__ __align__(16) KvSmem<D, NW> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hl = lane >> 5;
    const int bg = blockIdx.x % BG;
    const int kblk = blockIdx.x / BG;                      // earliest keys (most queries) first
    const int b = bg / Hkv, g = bg % Hkv;
    const int G = Hq / Hkv;
    const float c = kLog2e / sqrtf((float)D);
    const float scale = 1.0f / sqrtf((float)D);
    const int nQT = (S + kTile - 1) / kTile;

    const int kt = kblk * NW + wave;                       // this wave's key tile
    const int j0 = kt * kTile;
    const bool wave_ok = j0 < S;
    const int qt_lo = kblk * NW;
    const int last_key = min(S - 1, (kblk * NW + NW) * kTile - 1);
    const int qt_hi = (int)min((long)nQT - 1, ((long)last_key + W - 1) / kTile);

    // K and V rows of this wave's tile into its own LDS rows (B operands of S
    // and dP: lane = key, dims 16ks + 8hl), read back every query tile.
    {
        const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kTile, S - j0)));
        const uint32_t rs = (uint32_t)Hkv * D * 2;
        const size_t base = (((size_t)b * S + min(j0, S - 1)) * Hkv + g) * D;
        const rsrc_t kr = make_rsrc(k + base, (uint32_t)rows * rs);
        const rsrc_t vr = make_rsrc(v + base, (uint32_t)rows * rs);
        constexpr int CH = D / 8;
#pragma unroll
        for (int u = 0; u < kTile * CH / 64; ++u) {
            const int item = lane + 64 * u, row = item / CH, ch = item % CH;
            *(bf16x8 *)&sm.kw[wave][row][8 * ch] = buf_load16(kr, row * rs + 16 * ch, 0);
            *(bf16x8 *)&sm.vw[wave][row][8 * ch] = buf_load16(vr, row * rs + 16 * ch, 0);
        }
    }
    const int frag_off = (int)(((const char *)&sm.kw[wave][lq][8 * hl]) - (const char *)&sm);
    f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        dka[dt] = zero16();
        dva[dt] = zero16();
    }
    // Flat pipeline over (head, query tile) pairs n: while pair n computes
    // from buffer n&1, pair n+1 is in the other buffer and pair n+2 is in
    // flight in registers.  One barrier per pair.
    const int NQ = qt_hi - qt_lo + 1, N = G * NQ;
    KvStager<D, NT> st;
    auto stage_load = [&](int n) {
        st.load(q, dout, lse, dsum, b, g * G + n / NQ, (qt_lo + n % NQ) * kTile, S, Hq, tid);
    };
    stage_load(0);
    st.store(sm, 0, tid);
    if (N > 1) {
        stage_load(1);
        st.store(sm, 1, tid);
    }
    if (N > 2) stage_load(2);
    lds_barrier();

    for (int n = 0; n < N; ++n) {
        const int buf = n & 1;
        const int qt = qt_lo + n % NQ;
        const int r0 = qt * kTile;
        // Does this wave's key tile see any row of the query tile?
        const bool active = wave_ok && qt >= kt && (qt - kt) * kTile < W + kTile - 1;
        if (active) {                                      // wave-uniform
            // Re-read K/V fragments from LDS every pair (an opaque offset keeps
            // the compiler from hoisting 64 registers' worth of them).
            int fo = frag_off;
            asm volatile("" : "+v"(fo));
            const bf16 *kfrag = (const bf16 *)((const char *)&sm + fo);
            const bf16 *vfrag = kfrag + (sizeof(sm.kw) / sizeof(bf16));
            const bf16 *qrow = &sm.q[buf][score_row_key(lq)][8 * hl];
            const bf16 *grow = &sm.g[buf][score_row_key(lq)][8 * hl];
            f32x16 s = mfma32(*(const bf16x8 *)qrow, *(const bf16x8 *)kfrag, zero16());
            f32x16 dp = mfma32(*(const bf16x8 *)grow, *(const bf16x8 *)vfrag, zero16());
#pragma unroll
            for (int ks = 1; ks < D / 16; ++ks) {
                s = mfma32(*(const bf16x8 *)(qrow + 16 * ks), *(const bf16x8 *)(kfrag + 16 * ks), s);
                dp = mfma32(*(const bf16x8 *)(grow + 16 * ks), *(const bf16x8 *)(vfrag + 16 * ks), dp);
            }
            // rows i = r0 + perm_row(r, hl), key j = j0 + lq: visible iff j <= i < j + W
            const bool masked = qt == kt || (qt * kTile + kTile - 1) - W >= j0;
            f32x16 &p = s, &ds = dp;                       // computed in place
            {
                f32x4 l2v[4], ddv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int row = 16 * (u >> 1) + 8 * hl + 4 * (u & 1);
                    l2v[u] = *(const f32x4 *)&sm.l2[buf][row];
                    ddv[u] = *(const f32x4 *)&sm.dd[buf][row];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = s[r];
                    if (masked) {
                        const int dij = (r0 + perm_row(r, hl)) - (j0 + lq);
                        x = (dij >= 0 && dij < W) ? x : -INFINITY;
                    }
                    const float l2r = l2v[r >> 2][r & 3], ddr = ddv[r >> 2][r & 3];
                    const float pr = __builtin_amdgcn_exp2f(fmaf(x, c, -l2r));
                    ds[r] = pr * (dp[r] - ddr);
                    p[r] = pr;
                }
            }
            const bf16x8 pa = pack8(p, 0), pb = pack8(p, 1);
            const bf16x8 da = pack8(ds, 0), db = pack8(ds, 1);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                dva[dt] = mfma32(*(const bf16x8 *)&sm.gt[buf][32 * dt + lq][8 * hl], pa, dva[dt]);
                dva[dt] = mfma32(*(const bf16x8 *)&sm.gt[buf][32 * dt + lq][16 + 8 * hl], pb, dva[dt]);
                dka[dt] = mfma32(*(const bf16x8 *)&sm.qt[buf][32 * dt + lq][8 * hl], da, dka[dt]);
                dka[dt] = mfma32(*(const bf16x8 *)&sm.qt[buf][32 * dt + lq][16 + 8 * hl], db, dka[dt]);
            }
        }
        lds_barrier();                                     // buffer n&1 released
        if (n + 2 < N) {
            st.store(sm, buf, tid);                        // pair n+2 into the freed buffer
            if (n + 3 < N) stage_load(n + 3);
        }
    }

    if (wave_ok && j0 + lq < S) {
        const size_t off = (((size_t)b * S + j0 + lq) * Hkv + g) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 xk, xv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xk[e] = (bf16)(dka[dt][4 * jj + e] * scale);
                    xv[e] = (bf16)dva[dt][4 * jj + e];
                }
                *(bf16x4 *)(dk + off + 32 * dt + 8 * jj + 4 * hl) = xk;
                *(bf16x4 *)(dv + off + 32 * dt + 8 * jj + 4 * hl) = xv;
            }
    }
}

template <int D, int NW>
hipError_t launch_dq(const BackwardArgs &a, hipStream_t stream) {
    const int BG = a.B * a.Hkv;
    const int NB = (a.S + kTile - 1) / kTile;
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW>), dim3((unsigned)((long)BG * NB)), dim3(NW * 64), 0,
                       stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                       (const bf16 *)a.dout, a.lse, a.ws_dsum, (bf16 *)a.dq, a.S, a.Hq, a.Hkv,
                       a.window, BG, NB);
    return hipGetLastError();
}

constexpr int kKvWaves = 4;        // key tiles per dk/dv work-group

template <int D>
hipError_t launch_dkdv(const BackwardArgs &a, hipStream_t stream) {
    const int BG = a.B * a.Hkv;
    const int nKT = (a.S + kTile - 1) / kTile;
    const int nblk = (nKT + kKvWaves - 1) / kKvWaves;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kKvWaves>), dim3((unsigned)((long)BG * nblk)),
                       dim3(kKvWaves * 64), 0, stream, (const bf16 *)a.q, (const bf16 *)a.k,
                       (const bf16 *)a.v, (const bf16 *)a.dout, a.lse, a.ws_dsum, (bf16 *)a.dk,
                       (bf16 *)a.dv, a.S, a.Hq, a.Hkv, a.window, BG);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BackwardArgs &a, hipStream_t stream) {
    hipError_t e;
    switch (waves_for_group(a.Hq / a.Hkv)) {
    case 8: e = launch_dq<D, 8>(a, stream); break;
    case 4: e = launch_dq<D, 4>(a, stream); break;
    case 2: e = launch_dq<D, 2>(a, stream); break;
    default: e = launch_dq<D, 1>(a, stream); break;
    }
    if (e != hipSuccess) return e;
    return launch_dkdv<D>(a, stream);
}

}  // namespace

hipError_t launch_backward_bf16(const BackwardArgs &a, hipStream_t stream) {
    hipError_t e = launch_backward_pre(a, stream, true);
    if (e != hipSuccess) return e;
    return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace swa
