/*
 * Main program of the sanitizer build of the CPU oracle (test infrastructure).
 *
 * tests/test_oracle_sanitize.py compiles this file together with
 * oracle/mate_oracle.c under -fsanitize=address,undefined and runs it. Every
 * oracle entry point is called on small ragged shapes, several threads, with
 * and without review tokens, so that the address and undefined-behaviour
 * checkers see every loop and buffer of the oracle. The results are also
 * checked against closed forms that hold for any input:
 *   - each scan order is a bijection of the tokens, and the flip reverses it;
 *   - a reorder followed by its inverse gives the input back;
 *   - a 1x1x1 pool gives every token as its own review token;
 *   - B = 0 makes both scan directions return D x, so y = 2 D x (the SSD scan
 *     and the selective scan);
 *   - a one-token grid gives y = 2 (dt (C . B) x + D x);
 *   - a 1x1x1 attention window gives o = v, and its backward dv = dout,
 *     dq = dk = 0;
 *   - the scan's backward satisfies <dx, x> = <dy, y> (y is linear in x).
 * Prints "ALL OK" and exits 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_rms_sequence(int64_t T, int64_t H, int64_t W, int order, int flip, int64_t *seq);
int oracle_rms_reorder(const uint8_t *src, uint8_t *dst, int64_t batch, int64_t T, int64_t H, int64_t W,
                       int64_t row_bytes, int order, int flip, int inverse);
int oracle_review_pool(const float *src, int64_t T, int64_t H, int64_t W, int64_t C, int pt, int ph, int pw,
                       int order, double *out);
int oracle_bissd(const float *x, const float *B, const float *C, const float *dt, const float *A, const float *D,
                 int64_t batch, int64_t T, int64_t H, int64_t W, int nheads, int P, int S, int G, int order,
                 int pool_t, int pool_h, int pool_w, int head_lo, int head_hi, int nthreads, double *y);
int oracle_bissd_backward(const float *x, const float *B, const float *C, const float *dt, const float *A,
                          const float *D, const float *dy, int64_t batch, int64_t T, int64_t H, int64_t W,
                          int nheads, int P, int S, int G, int order, int pool_t, int pool_h, int pool_w,
                          int head_lo, int head_hi, int nthreads, double *dx, double *dB, double *dC, double *ddt,
                          double *dA, double *dD);
int oracle_biscan1(const float *x, const float *B, const float *C, const float *dt, const float *A, const float *D,
                   int64_t batch, int64_t T, int64_t H, int64_t W, int nch, int S, int order, int pool_t,
                   int pool_h, int pool_w, int ch_lo, int ch_hi, int nthreads, double *y);
int oracle_tesa_region_counts(int64_t T, int64_t H, int64_t W, int wt, int wh, int ww, int st, int sh, int sw,
                              int64_t *counts3);
int oracle_tesa(const float *q, const float *k, const float *v, int64_t batch, int64_t T, int64_t H, int64_t W,
                int nheads, int d, int wt, int wh, int ww, int st, int sh, int sw, double scale, int head_lo,
                int head_hi, const int64_t *regions, int64_t nregions, int nthreads, double *o);
int oracle_tesa_backward(const float *q, const float *k, const float *v, const float *dout, int64_t batch,
                         int64_t T, int64_t H, int64_t W, int nheads, int d, int wt, int wh, int ww, int st, int sh,
                         int sw, double scale, int head_lo, int head_hi, const int64_t *regions, int64_t nregions,
                         int nthreads, double *dq, double *dk, double *dv);

static int failures = 0;

#define CHECK(cond, ...)                                                                                       \
    do {                                                                                                       \
        if (!(cond)) {                                                                                         \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);                                               \
            fprintf(stderr, __VA_ARGS__);                                                                      \
            fprintf(stderr, "\n");                                                                             \
            ++failures;                                                                                        \
        }                                                                                                      \
    } while (0)

/* Deterministic values in (-1, 1) (a 64-bit LCG, high bits). */
static uint64_t lcg = 0x9e3779b97f4a7c15ull;
static float rnd(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((double)(lcg >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}
static float *rnd_array(size_t n, float lo, float hi)
{
    float *a = (float *)malloc(sizeof(float) * n);
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * 0.5f * (rnd() + 1.0f);
    return a;
}

static int close_to(double a, double b, double tol) { return fabs(a - b) <= tol * (1.0 + fabs(b)); }

static void check_rms(void)
{
    const int64_t grids[][3] = {{1, 1, 1}, {2, 3, 5}, {3, 4, 2}, {5, 1, 7}};
    for (size_t gi = 0; gi < sizeof(grids) / sizeof(grids[0]); ++gi) {
        const int64_t T = grids[gi][0], H = grids[gi][1], W = grids[gi][2], N = T * H * W;
        int64_t *seq = (int64_t *)malloc(sizeof(int64_t) * N), *rev = (int64_t *)malloc(sizeof(int64_t) * N);
        char *seen = (char *)calloc((size_t)N, 1);
        for (int order = 0; order <= 4; ++order) {
            CHECK(oracle_rms_sequence(T, H, W, order, 0, seq) == 0, "rms_sequence order %d", order);
            CHECK(oracle_rms_sequence(T, H, W, order, 1, rev) == 0, "rms_sequence flip order %d", order);
            memset(seen, 0, (size_t)N);
            for (int64_t i = 0; i < N; ++i) {
                CHECK(seq[i] >= 0 && seq[i] < N && !seen[seq[i]], "order %d not a bijection", order);
                if (seq[i] >= 0 && seq[i] < N) seen[seq[i]] = 1;
                CHECK(rev[i] == seq[N - 1 - i], "flip of order %d is not the reversal", order);
            }
            /* reorder then inverse reorder, batch 2, odd row size */
            const int64_t row = 7, batch = 2;
            uint8_t *src = (uint8_t *)malloc((size_t)(batch * N * row)), *mid = (uint8_t *)malloc((size_t)(batch * N * row)),
                    *back = (uint8_t *)malloc((size_t)(batch * N * row));
            for (int64_t e = 0; e < batch * N * row; ++e) src[e] = (uint8_t)(e * 31 + 7);
            CHECK(oracle_rms_reorder(src, mid, batch, T, H, W, row, order, 1, 0) == 0, "reorder");
            CHECK(oracle_rms_reorder(mid, back, batch, T, H, W, row, order, 1, 1) == 0, "inverse reorder");
            CHECK(memcmp(src, back, (size_t)(batch * N * row)) == 0, "reorder round trip, order %d", order);
            free(src);
            free(mid);
            free(back);
        }
        free(seq);
        free(rev);
        free(seen);
    }
}

static void check_pool(void)
{
    const int64_t T = 2, H = 3, W = 5, C = 3, N = T * H * W;
    float *x = rnd_array((size_t)(N * C), -1, 1);
    double *out = (double *)malloc(sizeof(double) * N * C);
    int64_t *seq = (int64_t *)malloc(sizeof(int64_t) * N);
    for (int order = 0; order <= 4; ++order) {
        CHECK(oracle_review_pool(x, T, H, W, C, 1, 1, 1, order, out) == 0, "pool");
        oracle_rms_sequence(T, H, W, order, 0, seq);
        for (int64_t j = 0; j < N; ++j)
            for (int64_t c = 0; c < C; ++c)
                CHECK(out[j * C + c] == (double)x[seq[j] * C + c], "1x1x1 pool is not the identity");
    }
    double *p2 = (double *)malloc(sizeof(double) * 5 * C);
    CHECK(oracle_review_pool(x, T, H, W, C, 2, 3, 1, 0, p2) == 0, "2x3x1 pool");
    CHECK(oracle_review_pool(x, T, H, W, C, 2, 2, 1, 0, p2) != 0, "a pool that does not divide the grid is rejected");
    free(p2);
    free(x);
    free(out);
    free(seq);
}

/* B = 0: y = 2 D x, both scans, with review tokens; a one-token grid: the closed form. */
static void check_scans(void)
{
    const int64_t batch = 2, T = 3, H = 2, W = 5, N = T * H * W;
    const int nh = 4, P = 3, S = 5, G = 2;
    float *x = rnd_array((size_t)(batch * N * nh * P), -1, 1);
    float *Bz = (float *)calloc((size_t)(batch * N * G * S), sizeof(float));
    float *Cm = rnd_array((size_t)(batch * N * G * S), -1, 1);
    float *dt = rnd_array((size_t)(batch * N * nh), 0.05f, 1.0f);
    float *A = rnd_array((size_t)nh, -2.0f, -0.5f), *D = rnd_array((size_t)nh, -1, 1);
    double *y = (double *)malloc(sizeof(double) * batch * N * nh * P);
    for (int order = 0; order <= 4; ++order) {
        CHECK(oracle_bissd(x, Bz, Cm, dt, A, D, batch, T, H, W, nh, P, S, G, order, 3, 1, 5, 1, 4, 3, y) == 0, "bissd");
        for (int64_t t = 0; t < batch * N; ++t)
            for (int h = 1; h < 4; ++h)
                for (int p = 0; p < P; ++p)
                    CHECK(close_to(y[(t * 3 + (h - 1)) * P + p], 2.0 * D[h] * x[(t * nh + h) * P + p], 1e-12),
                          "bissd with B = 0 is not 2 D x");
    }
    free(y);
    /* selective scan: A per (channel, state), B = 0 */
    const int nch = 6, S1 = 4;
    float *x1 = rnd_array((size_t)(batch * N * nch), -1, 1), *dt1 = rnd_array((size_t)(batch * N * nch), 0.05f, 1.0f);
    float *A1 = rnd_array((size_t)(nch * S1), -2.0f, -0.5f), *D1 = rnd_array((size_t)nch, -1, 1);
    float *B1 = (float *)calloc((size_t)(batch * N * S1), sizeof(float)), *C1 = rnd_array((size_t)(batch * N * S1), -1, 1);
    double *y1 = (double *)malloc(sizeof(double) * batch * N * nch);
    for (int order = 0; order <= 4; ++order) {
        CHECK(oracle_biscan1(x1, B1, C1, dt1, A1, D1, batch, T, H, W, nch, S1, order, 1, 2, 5, 0, nch, 3, y1) == 0,
              "biscan1");
        for (int64_t e = 0; e < batch * N * nch; ++e)
            CHECK(close_to(y1[e], 2.0 * D1[e % nch] * x1[e], 1e-12), "biscan1 with B = 0 is not 2 D x");
    }
    /* one token: each direction sees h = dt x B^T, so y = 2 (dt (C . B) x + D x) */
    float *Bm = rnd_array((size_t)(G * S), -1, 1);
    double *y2 = (double *)malloc(sizeof(double) * nh * P);
    CHECK(oracle_bissd(x, Bm, Cm, dt, A, D, 1, 1, 1, 1, nh, P, S, G, 2, 0, 0, 0, 0, nh, 2, y2) == 0, "one-token bissd");
    for (int h = 0; h < nh; ++h) {
        const int g = h / (nh / G);
        double cb = 0.0;
        for (int s = 0; s < S; ++s) cb += (double)Cm[g * S + s] * (double)Bm[g * S + s];
        for (int p = 0; p < P; ++p)
            CHECK(close_to(y2[h * P + p], 2.0 * ((double)dt[h] * cb * x[h * P + p] + (double)D[h] * x[h * P + p]), 1e-12),
                  "one-token bissd");
    }
    free(x); free(Bz); free(Cm); free(dt); free(A); free(D); free(Bm); free(y2);
    free(x1); free(dt1); free(A1); free(D1); free(B1); free(C1); free(y1);
}

/* The scan's backward on a ragged shape with review tokens, more positions than one checkpoint block, a head
 * range and several threads; y is linear in x, so <dx, x> = <dy, y>. */
static void check_scan_backward(void)
{
    const int64_t batch = 2, T = 4, H = 9, W = 10, N = T * H * W; /* 360 positions + 45 review tokens */
    const int nh = 3, P = 2, S = 3, G = 1, lo = 1, hi = 3, nr = hi - lo;
    float *x = rnd_array((size_t)(batch * N * nh * P), -1, 1), *dy = rnd_array((size_t)(batch * N * nh * P), -1, 1);
    float *Bm = rnd_array((size_t)(batch * N * G * S), -1, 1), *Cm = rnd_array((size_t)(batch * N * G * S), -1, 1);
    float *dt = rnd_array((size_t)(batch * N * nh), 0.05f, 0.5f);
    float *A = rnd_array((size_t)nh, -1.0f, -0.2f), *D = rnd_array((size_t)nh, -1, 1);
    double *y = (double *)malloc(sizeof(double) * batch * N * nr * P);
    double *dx = (double *)malloc(sizeof(double) * batch * N * nr * P), *ddt = (double *)malloc(sizeof(double) * batch * N * nr);
    double *dB = (double *)malloc(sizeof(double) * batch * N * G * S), *dC = (double *)malloc(sizeof(double) * batch * N * G * S);
    double dA[3], dD[3];
    for (int order = 0; order <= 4; order += 2) {
        CHECK(oracle_bissd(x, Bm, Cm, dt, A, D, batch, T, H, W, nh, P, S, G, order, 2, 3, 5, lo, hi, 3, y) == 0, "bissd");
        CHECK(oracle_bissd_backward(x, Bm, Cm, dt, A, D, dy, batch, T, H, W, nh, P, S, G, order, 2, 3, 5, lo, hi, 3, dx,
                                    dB, dC, ddt, dA, dD) == 0,
              "bissd backward");
        double lhs = 0.0, rhs = 0.0;
        for (int64_t t = 0; t < batch * N; ++t)
            for (int h = lo; h < hi; ++h)
                for (int p = 0; p < P; ++p) {
                    lhs += dx[(t * nr + (h - lo)) * P + p] * x[(t * nh + h) * P + p];
                    rhs += (double)dy[(t * nh + h) * P + p] * y[(t * nr + (h - lo)) * P + p];
                }
        CHECK(close_to(lhs, rhs, 1e-10), "backward adjoint identity, order %d: %g vs %g", order, lhs, rhs);
    }
    free(x); free(dy); free(Bm); free(Cm); free(dt); free(A); free(D); free(y); free(dx); free(ddt); free(dB); free(dC);
}

/* Unit windows: o = v and the backward passes dout to dv; shifted ragged windows run through. */
static void check_tesa(void)
{
    const int64_t batch = 2, T = 3, H = 4, W = 6, N = T * H * W;
    const int nh = 3, d = 5;
    const size_t n = (size_t)(batch * N * nh * d);
    float *q = rnd_array(n, -1, 1), *k = rnd_array(n, -1, 1), *v = rnd_array(n, -1, 1), *dout = rnd_array(n, -1, 1);
    double *o = (double *)malloc(sizeof(double) * n), *dq = (double *)malloc(sizeof(double) * n),
           *dk = (double *)malloc(sizeof(double) * n), *dv = (double *)malloc(sizeof(double) * n);
    CHECK(oracle_tesa(q, k, v, batch, T, H, W, nh, d, 1, 1, 1, 0, 0, 0, 0.0, 0, nh, NULL, 0, 3, o) == 0, "tesa");
    for (size_t e = 0; e < n; ++e) CHECK(close_to(o[e], v[e], 1e-15), "unit window is not v");
    CHECK(oracle_tesa_backward(q, k, v, dout, batch, T, H, W, nh, d, 1, 1, 1, 0, 0, 0, 0.0, 0, nh, NULL, 0, 3, dq, dk,
                               dv) == 0,
          "tesa backward");
    for (size_t e = 0; e < n; ++e)
        CHECK(close_to(dv[e], dout[e], 1e-15) && dq[e] == 0.0 && dk[e] == 0.0, "unit-window backward");
    /* shifted windows with ragged edge regions, a region subset, every head range */
    int64_t counts[3];
    CHECK(oracle_tesa_region_counts(T, H, W, 3, 2, 3, 1, 1, 2, counts) == 0, "region counts");
    const int64_t nreg = counts[0] * counts[1] * counts[2];
    int64_t regions[2] = {0, nreg - 1};
    CHECK(oracle_tesa(q, k, v, batch, T, H, W, nh, d, 3, 2, 3, 1, 1, 2, 0.0, 1, 3, regions, 2, 4, o) == 0, "tesa subset");
    CHECK(oracle_tesa(q, k, v, batch, T, H, W, nh, d, 3, 2, 3, 1, 1, 2, 0.0, 0, nh, NULL, 0, 4, o) == 0, "tesa shifted");
    for (size_t e = 0; e < n; ++e) CHECK(isfinite(o[e]), "tesa output not finite");
    CHECK(oracle_tesa_backward(q, k, v, dout, batch, T, H, W, nh, d, 3, 2, 3, 1, 1, 2, 0.0, 0, nh, NULL, 0, 4, dq, dk,
                               dv) == 0,
          "tesa backward shifted");
    CHECK(oracle_tesa(q, k, v, batch, T, H, W, nh, d, 3, 2, 3, 3, 1, 2, 0.0, 0, nh, NULL, 0, 4, o) != 0,
          "a shift outside [0, window) is rejected");
    free(q); free(k); free(v); free(dout); free(o); free(dq); free(dk); free(dv);
}

int main(void)
{
    check_rms();
    check_pool();
    check_scans();
    check_scan_backward();
    check_tesa();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ALL OK\n");
    return 0;
}
