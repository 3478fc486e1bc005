/*
 * oracle.c -- plain fp64 CPU reference for causal attention with a sliding
 * window and a learnable per-head sink.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (one query row, one head):
 *
 *   Sources (page title, section):
 *   - "MiMo-V2-Flash Technical Report" digest, 前置知识 / 注意力sink偏置
 *     (attention-sink bias): every head adds a learnable term s_sink to the
 *     softmax denominator, i.e. a virtual sink token that can take attention
 *     mass away from the real tokens.  The virtual token has no value vector
 *     (it contributes nothing to the numerator).
 *   - same page, 前置知识 / 混合注意力机制 (hybrid attention) and 核心方法
 *     (core method): sliding-window layers see only a local window of
 *     128 tokens; global layers see the whole (causal) prefix.
 *   - "小米罗福莉：MiMo-V2.5如何做到又快又强又便宜？| ICML 2026", §02 of
 *     the talk: grouped-query attention is used throughout.
 *
 *   For query row i of head h (KV head g = h / (Hq/Hkv)), with key set K_i:
 *     x_j  = (1/sqrt(D)) * sum_d q[i,h,d] * k[j,g,d]           j in K_i
 *     M    = max(s_h, max_j x_j)
 *     Z    = sum_j exp(x_j - M)
 *     E    = exp(s_h - M)            (0 when s_h = -inf)
 *     out  = sum_j exp(x_j - M) * v[j,g,:] / (Z + E)
 *     lse  = M + log(Z + E)
 *   An empty key set leaves only the sink: out = 0, lse = s_h.
 *
 * Everything is evaluated directly in double precision from the exact input
 * values: no tiling, no online rescaling, no reordering.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Attention of one query row over n key rows given by pointer arrays. */
static void attend_row(const double *qrow, int64_t D, double sink,
                       const double *const *krows, const double *const *vrows,
                       int64_t n, double *x, double *out_row, double *lse_out)
{
    const double scale = 1.0 / sqrt((double)D);
    double M = sink;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += qrow[d] * krows[j][d];
        x[j] = scale * dot;
        if (x[j] > M)
            M = x[j];
    }
    for (int64_t d = 0; d < D; ++d)
        out_row[d] = 0.0;
    if (n == 0) {
        /* Only the virtual sink token is left; it has no value vector. */
        *lse_out = sink;
        return;
    }
    double Z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        const double w = exp(x[j] - M);
        Z += w;
        for (int64_t d = 0; d < D; ++d)
            out_row[d] += w * vrows[j][d];
    }
    const double E = isinf(sink) && sink < 0 ? 0.0 : exp(sink - M);
    for (int64_t d = 0; d < D; ++d)
        out_row[d] /= (Z + E);
    *lse_out = M + log(Z + E);
}

/*
 * Query rows r = 0..R-1 of batch qb[r], every head, over the key positions
 * lo[r]..hi[r] (inclusive; empty when hi < lo) of k/v laid out [B, N, Hkv, D].
 *   q   [R, Hq, D]     out [R, Hq, D]     lse [R, Hq]     sink [Hq]
 * Used for sliding-window prefill (lo = max(0, i-W+1), hi = i), for global
 * causal attention (lo = 0, hi = position of the query) and for sampled rows.
 */
void oracle_attend_rows(const double *q, const int64_t *qb, const int64_t *lo,
                        const int64_t *hi, const double *k, const double *v,
                        const double *sink, double *out, double *lse,
                        int64_t R, int64_t N, int64_t Hq, int64_t Hkv, int64_t D)
{
    const int64_t G = Hq / Hkv;
#pragma omp parallel
    {
        double *x = NULL;
        const double **kr = NULL, **vr = NULL;
        int64_t cap = 0;
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int64_t r = 0; r < R; ++r) {
            for (int64_t h = 0; h < Hq; ++h) {
                const int64_t g = h / G;
                const int64_t first = lo[r] < 0 ? 0 : lo[r];
                const int64_t last = hi[r] >= N ? N - 1 : hi[r];
                const int64_t n = last >= first ? last - first + 1 : 0;
                if (n > cap) {
                    cap = n;
                    x = (double *)realloc(x, (size_t)cap * sizeof(double));
                    kr = (const double **)realloc(kr, (size_t)cap * sizeof(double *));
                    vr = (const double **)realloc(vr, (size_t)cap * sizeof(double *));
                }
                for (int64_t j = 0; j < n; ++j) {
                    const int64_t pos = first + j;
                    const int64_t off = ((qb[r] * N + pos) * Hkv + g) * D;
                    kr[j] = k + off;
                    vr[j] = v + off;
                }
                attend_row(q + (r * Hq + h) * D, D, sink[h], kr, vr, n, x,
                           out + (r * Hq + h) * D, lse + r * Hq + h);
            }
        }
        free(x);
        free(kr);
        free(vr);
    }
}

/*
 * Decode over a fixed ring of W slots per (sequence, KV head): the key of
 * absolute position P lives in slot P mod W.  Sources: the pwwt.cn article
 * on MiMo-V2-Flash, §1.1 Hybrid Attention (a sliding-window layer keeps a
 * fixed-size KV cache, O(W) memory); "小米罗福莉 ... ICML 2026", Q&A on RoPE
 * (positions keep increasing as the window slides, so cached keys carry
 * absolute positions); the technical-report digest, 前置知识 / 多token预测
 * (MTP draft tokens are verified by the main model in one parallel pass).
 *
 *   q [B, T, Hq, D]   kc, vc [B, Hkv, W, D]   out [B, T, Hq, D]   lse [B, T, Hq]
 *   cache_len [B]: L_b = tokens written so far, including the T new ones.
 * The ring has W slots (position P in slot P mod W); the attention window is
 * Wnd keys (Wnd <= W).  Query t sits at position p = L - T + t and sees the
 * positions max(0, L-W, p-Wnd+1) .. p: everything older than L-W has been
 * overwritten, and the window reaches back Wnd-1 positions.  With Wnd = W
 * the bound is max(0, L-W); a ring of Wnd + T - 1 slots gives every query
 * its full window (none of them needs a position older than L-W).
 */
void oracle_ring_decode(const double *q, const double *kc, const double *vc,
                        const double *sink, const int64_t *cache_len,
                        double *out, double *lse, int64_t B, int64_t T,
                        int64_t Hq, int64_t Hkv, int64_t W, int64_t D, int64_t Wnd)
{
    const int64_t G = Hq / Hkv;
#pragma omp parallel
    {
        double *x = (double *)malloc((size_t)W * sizeof(double));
        const double **kr = (const double **)malloc((size_t)W * sizeof(double *));
        const double **vr = (const double **)malloc((size_t)W * sizeof(double *));
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t t = 0; t < T; ++t) {
                for (int64_t h = 0; h < Hq; ++h) {
                    const int64_t g = h / G;
                    const int64_t L = cache_len[b];
                    const int64_t p = L - T + t;
                    const int64_t oldest = L - W > 0 ? L - W : 0;
                    const int64_t first = p - Wnd + 1 > oldest ? p - Wnd + 1 : oldest;
                    int64_t n = 0;
                    for (int64_t P = first; P <= p; ++P) {
                        const int64_t slot = P % W;
                        const int64_t off = ((b * Hkv + g) * W + slot) * D;
                        kr[n] = kc + off;
                        vr[n] = vc + off;
                        ++n;
                    }
                    const int64_t row = (b * T + t) * Hq + h;
                    attend_row(q + row * D, D, sink[h], kr, vr, n, x,
                               out + row * D, lse + row);
                }
            }
        }
        free(x);
        free(kr);
        free(vr);
    }
}

/*
 * Gradients of causal sliding-window (or, with W >= S, global causal)
 * attention with a sink, for an upstream gradient dout.  The sink s_h is a
 * learnable per-head parameter (technical-report digest, 前置知识 /
 * 注意力sink偏置), so its gradient is part of the result.
 *
 *   q, dout, dq [B, S, Hq, D]    k, v, dk, dv [B, S, Hkv, D]
 *   sink, dsink [Hq]             row i sees positions max(0, i-W+1) .. i
 *
 * With the forward of one row written as
 *   x_j = scale q_i.k_j,  lse = log(e^{s_h} + sum_j e^{x_j}),
 *   P_j = e^{x_j - lse},  p_sink = e^{s_h - lse},  out_i = sum_j P_j v_j
 * and L = sum over rows and heads of dout_i . out_i, the chain rule gives
 *   dv_j  += P_j dout_i
 *   dP_j   = dout_i . v_j
 *   Dsum   = sum_j P_j dP_j         (the sink's value vector is zero)
 *   dx_j   = P_j (dP_j - Dsum)
 *   ds_h  += p_sink (0 - Dsum)
 *   dq_i  += scale dx_j k_j,    dk_j += scale dx_j q_i
 * Every row's forward is recomputed from the definition; dk and dv sum over
 * the query heads that share a KV head, dsink over sequences and rows.
 */
void oracle_attend_backward(const double *q, const double *k, const double *v,
                            const double *sink, const double *dout, double *dq,
                            double *dk, double *dv, double *dsink, int64_t B,
                            int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                            int64_t W)
{
    const int64_t G = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)D);
    double *ds_part = (double *)calloc((size_t)(B * Hq), sizeof(double));
    for (int64_t e = 0; e < B * S * Hq * D; ++e)
        dq[e] = 0.0;
    for (int64_t e = 0; e < B * S * Hkv * D; ++e) {
        dk[e] = 0.0;
        dv[e] = 0.0;
    }
#pragma omp parallel
    {
        double *x = (double *)malloc((size_t)S * sizeof(double));
        double *dp = (double *)malloc((size_t)S * sizeof(double));
        /* (b, g) pairs own disjoint rows of dk, dv and dq: no races. */
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t g = 0; g < Hkv; ++g) {
                for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                    const double s = sink[h];
                    for (int64_t i = 0; i < S; ++i) {
                        const int64_t lo = i - W + 1 > 0 ? i - W + 1 : 0;
                        const int64_t n = i - lo + 1;
                        const double *qi = q + ((b * S + i) * Hq + h) * D;
                        const double *gi = dout + ((b * S + i) * Hq + h) * D;
                        /* forward of the row: scores, max, log-sum-exp */
                        double M = s;
                        for (int64_t j = 0; j < n; ++j) {
                            const double *kj = k + ((b * S + lo + j) * Hkv + g) * D;
                            double dot = 0.0;
                            for (int64_t d = 0; d < D; ++d)
                                dot += qi[d] * kj[d];
                            x[j] = scale * dot;
                            if (x[j] > M)
                                M = x[j];
                        }
                        double Z = 0.0;
                        for (int64_t j = 0; j < n; ++j)
                            Z += exp(x[j] - M);
                        const double E = isinf(s) && s < 0 ? 0.0 : exp(s - M);
                        const double lse = M + log(Z + E);
                        /* dP_j = dout_i . v_j and Dsum = sum_j P_j dP_j */
                        double Dsum = 0.0;
                        for (int64_t j = 0; j < n; ++j) {
                            const double *vj = v + ((b * S + lo + j) * Hkv + g) * D;
                            double dot = 0.0;
                            for (int64_t d = 0; d < D; ++d)
                                dot += gi[d] * vj[d];
                            dp[j] = dot;
                            Dsum += exp(x[j] - lse) * dot;
                        }
                        const double p_sink = isinf(s) && s < 0 ? 0.0 : exp(s - lse);
                        ds_part[b * Hq + h] += p_sink * (0.0 - Dsum);
                        double *dqi = dq + ((b * S + i) * Hq + h) * D;
                        for (int64_t j = 0; j < n; ++j) {
                            const double P = exp(x[j] - lse);
                            const double dx = P * (dp[j] - Dsum);
                            const int64_t row = (b * S + lo + j) * Hkv + g;
                            const double *kj = k + row * D;
                            for (int64_t d = 0; d < D; ++d) {
                                dv[row * D + d] += P * gi[d];
                                dk[row * D + d] += scale * dx * qi[d];
                                dqi[d] += scale * dx * kj[d];
                            }
                        }
                    }
                }
            }
        }
        free(x);
        free(dp);
    }
    for (int64_t h = 0; h < Hq; ++h) {
        double t = 0.0;
        for (int64_t b = 0; b < B; ++b)
            t += ds_part[b * Hq + h];
        dsink[h] = t;
    }
    free(ds_part);
}

/* Rotary position embedding of n rows of H heads at absolute positions pos.
 * Source: "小米罗福莉：MiMo-V2.5如何做到又快又强又便宜？| ICML 2026", Q&A on
 * RoPE (positions keep increasing as the window slides: cached keys carry
 * their absolute positions).  Reading: the standard rotary embedding over
 * the whole head, dimension i paired with i + D/2, angle pos * theta^(-2i/D):
 *   y[i]       = x[i] cos(a) - x[i+D/2] sin(a)
 *   y[i + D/2] = x[i+D/2] cos(a) + x[i] sin(a)
 *   x, y [n, H, D]   pos [n]
 */
void oracle_rope(const double *x, const int64_t *pos, double *y, int64_t n, int64_t H,
                 int64_t D, double theta)
{
    const int64_t half = D / 2;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < half; ++i) {
            const double a = (double)pos[r] * pow(theta, -2.0 * (double)i / (double)D);
            const double cs = cos(a), sn = sin(a);
            for (int64_t h = 0; h < H; ++h) {
                const double *xr = x + (r * H + h) * D;
                double *yr = y + (r * H + h) * D;
                yr[i] = xr[i] * cs - xr[i + half] * sn;
                yr[i + half] = xr[i + half] * cs + xr[i] * sn;
            }
        }
}

/* Block maxima of the scaled logits of global causal attention.
 * Source: "小米罗福莉：MiMo-V2.5如何做到又快又强又便宜？| ICML 2026", §02
 * (High Sparse): later sparse layers select tokens by block from the
 * block-level scores the full-attention layer's FlashAttention pass produces.
 * Reading: the block score is the largest scaled logit x_ij = q_i . k_j /
 * sqrt(D) over the visible (row, key) pairs of the block -- the quantity the
 * pass already forms per tile -- in the units of the sink s_h; -inf when the
 * block has no visible pair.  Query blocks are 32 rows, key blocks bk keys;
 * queries at the end of the keys (row i at position S_kv - S_q + i).
 *   q [B,S_q,Hq,D], k [B,S_kv,Hkv,D] -> bmax [B, Hq, ceil(S_q/32), ceil(S_kv/bk)]
 */
void oracle_block_max(const double *q, const double *k, double *bmax, int64_t B,
                      int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D,
                      int64_t bk)
{
    const int64_t G = Hq / Hkv, nqb = (S_q + 31) / 32, nkb = (S_kv + bk - 1) / bk;
    const double scale = 1.0 / sqrt((double)D);
    const int64_t n = B * Hq * nqb * nkb;
    for (int64_t e = 0; e < n; ++e) bmax[e] = -INFINITY;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / G;
            double *blk = bmax + (b * Hq + h) * nqb * nkb;
            for (int64_t i = 0; i < S_q; ++i) {
                const int64_t pos = S_kv - S_q + i;
                const double *qi = q + ((b * S_q + i) * Hq + h) * D;
                for (int64_t j = 0; j <= pos; ++j) {
                    const double *kj = k + ((b * S_kv + j) * Hkv + g) * D;
                    double x = 0.0;
                    for (int64_t d = 0; d < D; ++d) x += qi[d] * kj[d];
                    x *= scale;
                    double *slot = blk + (i / 32) * nkb + j / bk;
                    if (x > *slot) *slot = x;
                }
            }
        }
}

/* Number of (query, key) pairs a causal window-W layer attends over S tokens:
 * enumerated one row at a time (used to check closed-form FLOP counts). */
int64_t oracle_count_window_pairs(int64_t S, int64_t W)
{
    int64_t total = 0;
    for (int64_t i = 0; i < S; ++i) {
        const int64_t lo = i - W + 1 > 0 ? i - W + 1 : 0;
        total += i - lo + 1;
    }
    return total;
}

/* Sets the threads later parallel regions use (n >= 1); timing only. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Threads an OpenMP parallel region of the oracle uses. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
