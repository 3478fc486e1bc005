/*
 * oracle_check.c -- runs every function of oracle/oracle.c on small inputs
 * with the edge cases the tests use (empty key sets, rings shorter than the
 * query block, window 1, window past the sequence, -inf sinks, GQA), built
 * with AddressSanitizer and UndefinedBehaviorSanitizer.  Besides memory and
 * UB errors (which abort), it checks identities that hold exactly:
 *   - V = 1:           out = 1 - exp(s - lse) in every element;
 *   - empty key set:   out = 0, lse = s;
 *   - ring decode of the newest position = the prefill's last row;
 *   - RoPE keeps the norm of every rotated pair;
 *   - pair counts:     W*S - W*(W-1)/2 for S >= W.
 * Exit status 0 when all hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_attend_rows(const double *q, const int64_t *qb, const int64_t *lo, const int64_t *hi,
                        const double *k, const double *v, const double *sink, double *out,
                        double *lse, int64_t R, int64_t N, int64_t Hq, int64_t Hkv, int64_t D);
void oracle_ring_decode(const double *q, const double *kc, const double *vc, const double *sink,
                        const int64_t *cache_len, double *out, double *lse, int64_t B, int64_t T,
                        int64_t Hq, int64_t Hkv, int64_t W, int64_t D, int64_t Wnd);
void oracle_attend_backward(const double *q, const double *k, const double *v, const double *sink,
                            const double *dout, double *dq, double *dk, double *dv, double *dsink,
                            int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t W);
void oracle_rope(const double *x, const int64_t *pos, double *y, int64_t n, int64_t H, int64_t D,
                 double theta);
void oracle_block_max(const double *q, const double *k, double *bmax, int64_t B, int64_t S_q,
                      int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t bk);
int64_t oracle_count_window_pairs(int64_t S, int64_t W);
void oracle_set_threads(int n);
int oracle_threads(void);

static int failures = 0;
#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #c);  \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static uint64_t state = 88172645463325252ull;
static double gauss(void) {          /* sum of uniforms: enough for a smoke test */
    double s = 0.0;
    for (int i = 0; i < 4; ++i) {
        state ^= state << 13; state ^= state >> 7; state ^= state << 17;
        s += (double)(state >> 11) / 9007199254740992.0;
    }
    return (s - 2.0) * 1.7;
}
static double *fill(size_t n, double value, int random) {
    double *p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = random ? gauss() : value;
    return p;
}

int main(void) {
    oracle_set_threads(2);
    CHECK(oracle_threads() >= 1);
    const int64_t B = 2, S = 40, Hq = 4, Hkv = 2, D = 8;
    double *q = fill(B * S * Hq * D, 0, 1), *k = fill(B * S * Hkv * D, 0, 1);
    double *ones = fill(B * S * Hkv * D, 1.0, 0), *v = fill(B * S * Hkv * D, 0, 1);
    double sink[4] = {0.3, -INFINITY, 5.0, -7.0};
    /* prefill rows for windows 1, 7, S and past S, plus empty rows (lo > hi) */
    const int64_t windows[4] = {1, 7, S, 3 * S};
    const int64_t R = B * S + 3;
    int64_t *qb = malloc(R * sizeof(int64_t)), *lo = malloc(R * sizeof(int64_t)),
            *hi = malloc(R * sizeof(int64_t));
    double *qr = malloc(R * Hq * D * sizeof(double)), *out = malloc(R * Hq * D * sizeof(double)),
           *lse = malloc(R * Hq * sizeof(double));
    for (int w = 0; w < 4; ++w) {
        for (int64_t r = 0; r < R; ++r) {
            const int64_t b = r < B * S ? r / S : r % B, i = r < B * S ? r % S : 5;
            qb[r] = b;
            hi[r] = r < B * S ? i : i - 10 - r;         /* the last 3 rows: empty */
            lo[r] = i - windows[w] + 1 > 0 ? i - windows[w] + 1 : 0;
            memcpy(qr + r * Hq * D, q + (b * S + i) * Hq * D, Hq * D * sizeof(double));
        }
        oracle_attend_rows(qr, qb, lo, hi, k, ones, sink, out, lse, R, S, Hq, Hkv, D);
        for (int64_t r = 0; r < R; ++r)
            for (int64_t h = 0; h < Hq; ++h) {
                const int empty = r >= B * S;
                const double l = lse[r * Hq + h];
                if (empty) CHECK(l == sink[h] || (isinf(l) && isinf(sink[h])));
                for (int64_t d = 0; d < D; ++d) {
                    const double o = out[(r * Hq + h) * D + d];
                    const double want = empty ? 0.0 : 1.0 - (isinf(sink[h]) ? 0.0 : exp(sink[h] - l));
                    CHECK(fabs(o - want) <= 1e-12);
                }
            }
    }
    /* ring decode: rings of W = 16 slots holding the last positions of the
       sequences; the newest query equals the full-window prefill row */
    {
        const int64_t W = 16, T = 3;
        const int64_t lens[2] = {S, 2};             /* sequence 1: fewer tokens than T */
        double *kc = fill(B * Hkv * W * D, NAN, 0), *vc = fill(B * Hkv * W * D, NAN, 0);
        for (int64_t b = 0; b < B; ++b)
            for (int64_t p = lens[b] - W > 0 ? lens[b] - W : 0; p < lens[b]; ++p)
                for (int64_t g = 0; g < Hkv; ++g)
                    for (int64_t d = 0; d < D; ++d) {
                        kc[((b * Hkv + g) * W + p % W) * D + d] = k[((b * S + p) * Hkv + g) * D + d];
                        vc[((b * Hkv + g) * W + p % W) * D + d] = v[((b * S + p) * Hkv + g) * D + d];
                    }
        double *qd = malloc(B * T * Hq * D * sizeof(double));
        for (int64_t b = 0; b < B; ++b)
            for (int64_t t = 0; t < T; ++t) {
                const int64_t p = lens[b] - T + t;
                memcpy(qd + (b * T + t) * Hq * D, q + (b * S + (p > 0 ? p : 0)) * Hq * D,
                       Hq * D * sizeof(double));
            }
        double *od = malloc(B * T * Hq * D * sizeof(double)), *ld = malloc(B * T * Hq * sizeof(double));
        for (int64_t wnd = 1; wnd <= W; wnd += 5) {
            oracle_ring_decode(qd, kc, vc, sink, lens, od, ld, B, T, Hq, Hkv, W, D, wnd);
            for (int64_t i = 0; i < B * T * Hq * D; ++i) CHECK(!isnan(od[i]));   /* unwritten slots unread */
        }
        oracle_ring_decode(qd, kc, vc, sink, lens, od, ld, B, T, Hq, Hkv, W, D, W);
        int64_t one_b = 0, one_lo = S - W, one_hi = S - 1;
        double pr[4 * 8], pl[4];
        oracle_attend_rows(q + (S - 1) * Hq * D, &one_b, &one_lo, &one_hi, k, v, sink, pr, pl, 1, S,
                           Hq, Hkv, D);
        for (int64_t h = 0; h < Hq; ++h) {
            CHECK(fabs(ld[(T - 1) * Hq + h] - pl[h]) <= 1e-12);
            for (int64_t d = 0; d < D; ++d)
                CHECK(fabs(od[((T - 1) * Hq + h) * D + d] - pr[h * D + d]) <= 1e-12);
        }
        free(kc); free(vc); free(qd); free(od); free(ld);
    }
    /* backward: finite results; a -inf sink has no gradient */
    {
        double *g = fill(B * S * Hq * D, 0, 1);
        double *dq = malloc(B * S * Hq * D * sizeof(double)), *dk = malloc(B * S * Hkv * D * sizeof(double)),
               *dv = malloc(B * S * Hkv * D * sizeof(double)), ds[4];
        for (int w = 0; w < 4; ++w) {
            oracle_attend_backward(q, k, v, sink, g, dq, dk, dv, ds, B, S, Hq, Hkv, D,
                                   windows[w] < S ? windows[w] : S);
            for (int64_t i = 0; i < B * S * Hq * D; ++i) CHECK(isfinite(dq[i]));
            for (int64_t i = 0; i < B * S * Hkv * D; ++i) CHECK(isfinite(dk[i]) && isfinite(dv[i]));
            CHECK(ds[1] == 0.0 && isfinite(ds[0]) && isfinite(ds[2]));
        }
        free(g); free(dq); free(dk); free(dv);
    }
    /* RoPE keeps pair norms; block maxima are finite or -inf */
    {
        int64_t pos[6] = {0, 1, 2, 1000, 1 << 20, (int64_t)1 << 40};
        double *x = fill(6 * Hq * D, 0, 1), *y = malloc(6 * Hq * D * sizeof(double));
        oracle_rope(x, pos, y, 6, Hq, D, 10000.0);
        for (int64_t r = 0; r < 6; ++r)
            for (int64_t h = 0; h < Hq; ++h)
                for (int64_t i = 0; i < D / 2; ++i) {
                    const double *a = x + (r * Hq + h) * D, *c = y + (r * Hq + h) * D;
                    const double n0 = a[i] * a[i] + a[i + D / 2] * a[i + D / 2];
                    const double n1 = c[i] * c[i] + c[i + D / 2] * c[i + D / 2];
                    CHECK(fabs(n0 - n1) <= 1e-9 * (1.0 + n0));
                }
        const int64_t Sq = 33, nqb = (Sq + 31) / 32;
        for (int64_t bk = 32; bk <= 96; bk += 32) {
            const int64_t nkb = (S + bk - 1) / bk;
            double *bm = malloc(B * Hq * nqb * nkb * sizeof(double));
            oracle_block_max(q + (S - Sq) * Hq * D, k, bm, 1, Sq, S, Hq, Hkv, D, bk);
            for (int64_t i = 0; i < Hq * nqb * nkb; ++i) CHECK(isfinite(bm[i]) || bm[i] == -INFINITY);
            free(bm);
        }
        free(x); free(y);
    }
    for (int64_t s = 0; s < 300; s += 37)
        for (int64_t w = 1; w < 200; w += 29) {
            const int64_t want = s >= w ? w * s - w * (w - 1) / 2 : s * (s + 1) / 2;
            CHECK(oracle_count_window_pairs(s, w) == want);
        }
    free(q); free(k); free(ones); free(v); free(qb); free(lo); free(hi); free(qr); free(out); free(lse);
    printf("oracle check: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
