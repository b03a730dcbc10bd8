/*
 * Plain CPU oracle for the MATE token-mixing core of LinGen.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously-correct
 * definition that the GPU library is checked against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it. It shares
 * no code, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * Everything is computed in double precision with explicit loops, in the
 * order the method is described:
 *
 *   - Rotary Major Scan (RMS) and the flipped sequence: four unroll orders of
 *     the T x H x W latent tensor that swap which axis is unrolled first
 *     (QbitAI article "LinGen ...", section "方法", the RMS paragraphs; the
 *     xllm-io review "LinGen: Towards High-Resolution Minute-Length ...",
 *     section 三 "MA-Branch" item 2, which names the four orders and the flip
 *     n_flip = T*H*W - n).
 *   - Zigzag scan, the alternative the pages compare RMS against (QbitAI
 *     article, section "方法"; xllm-io review, section 三 "MA-Branch" and
 *     Table 2, row "Zigzag"). The pages name it without defining it; it is
 *     read here as the snake path through the grid, whose consecutive tokens
 *     are always grid neighbours.
 *   - Review tokens: an average-pooled copy of the token tensor, unrolled in
 *     the same order and put in front of the sequence (forward) or, flipped,
 *     in front of the flipped sequence (xllm-io review, section 三 item 3;
 *     QbitAI article, review-token paragraph).
 *   - Bidirectional Mamba2 scan: the sequential state-space recurrence
 *     h_u = exp(dt_u A) h_{u-1} + dt_u x_u B_u^T, y_u = C_u^T h_u + D x_u,
 *     run over the forward sequence and over the flipped sequence, the two
 *     outputs summed (xllm-io review, section 三 item 1: Mamba2 alone gives the
 *     lower-triangular map, the bidirectional version the full map).
 *   - TESA: softmax attention restricted to 3D windows Tw x Sw x Sw whose
 *     partition is offset by a shift on alternate layers (xllm-io review,
 *     section 三 "TE-Branch"; nav.superapi summary, "TE-branch" bullet).
 *
 * Readings where the pages are silent (all documented in the design notes):
 *   - flip is the reversal i -> N-1-i;
 *   - pooling windows do not overlap (stride = kernel) and must divide the grid;
 *   - the recurrence starts from h = 0; outputs at review positions are dropped;
 *   - both directions share x, B, C, dt, A, D, so the sum carries 2 D x;
 *   - shifted windows: along each axis the region id of coordinate c is
 *     (c + w - s) div w, so edge regions are smaller and nothing wraps around;
 *   - attention scale is 1/sqrt(d) unless given; no position bias.
 *
 * Inputs are float32 arrays (values that may already be bf16-rounded; the
 * upcast to double is exact). Outputs are double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -2

/* ------------------------------------------------------------------------ */
/* Rotary Major Scan                                                         */
/* ------------------------------------------------------------------------ */

/* seq[i] = canonical index n(t,h,w) = (t*H + h)*W + w of the token at scan
 * position i.  Loops are written outermost first:
 *   order 0 spatial-row major:     for t, for h, for w
 *   order 1 spatial-column major:  for t, for w, for h
 *   order 2 temporal-row major:    for h, for w, for t
 *   order 3 temporal-column major: for w, for h, for t
 *   order 4 zigzag: frames in time order; frame t visits its rows h = 0..H-1
 *     on even t and H-1..0 on odd t; the path walks each row along w, turning
 *     round after every row it has covered (rows counted from the start of
 *     the path), so it never jumps: each step changes one coordinate by one.
 * flip != 0 reverses the sequence. */
int oracle_rms_sequence(int64_t T, int64_t H, int64_t W, int order, int flip, int64_t *seq)
{
    if (T <= 0 || H <= 0 || W <= 0 || order < 0 || order > 4 || !seq) return ORACLE_EINVAL;
    int64_t i = 0;
    if (order == 0) {
        for (int64_t t = 0; t < T; ++t)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t w = 0; w < W; ++w) seq[i++] = (t * H + h) * W + w;
    } else if (order == 1) {
        for (int64_t t = 0; t < T; ++t)
            for (int64_t w = 0; w < W; ++w)
                for (int64_t h = 0; h < H; ++h) seq[i++] = (t * H + h) * W + w;
    } else if (order == 2) {
        for (int64_t h = 0; h < H; ++h)
            for (int64_t w = 0; w < W; ++w)
                for (int64_t t = 0; t < T; ++t) seq[i++] = (t * H + h) * W + w;
    } else if (order == 3) {
        for (int64_t w = 0; w < W; ++w)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t t = 0; t < T; ++t) seq[i++] = (t * H + h) * W + w;
    } else {
        int64_t rows_done = 0;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t r = 0; r < H; ++r, ++rows_done) {
                const int64_t h = (t % 2 == 0) ? r : H - 1 - r;
                for (int64_t c = 0; c < W; ++c) {
                    const int64_t w = (rows_done % 2 == 0) ? c : W - 1 - c;
                    seq[i++] = (t * H + h) * W + w;
                }
            }
    }
    if (flip) {
        int64_t N = T * H * W;
        for (int64_t a = 0, b = N - 1; a < b; ++a, --b) {
            int64_t tmp = seq[a];
            seq[a] = seq[b];
            seq[b] = tmp;
        }
    }
    return ORACLE_OK;
}

/* Whole-row permutation of a [batch][T][H][W][row_bytes] byte tensor.
 * inverse == 0: dst[b][i] = src[b][seq[i]]  (canonical -> scan order)
 * inverse != 0: dst[b][seq[i]] = src[b][i]  (scan order -> canonical) */
int oracle_rms_reorder(const uint8_t *src, uint8_t *dst, int64_t batch, int64_t T, int64_t H,
                       int64_t W, int64_t row_bytes, int order, int flip, int inverse)
{
    if (!src || !dst || batch <= 0 || row_bytes <= 0) return ORACLE_EINVAL;
    int64_t N = T * H * W;
    int64_t *seq = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
    if (!seq) return ORACLE_ENOMEM;
    int rc = oracle_rms_sequence(T, H, W, order, flip, seq);
    if (rc) {
        free(seq);
        return rc;
    }
    for (int64_t b = 0; b < batch; ++b) {
        const uint8_t *s = src + b * N * row_bytes;
        uint8_t *d = dst + b * N * row_bytes;
        for (int64_t i = 0; i < N; ++i) {
            if (!inverse)
                memcpy(d + i * row_bytes, s + seq[i] * row_bytes, (size_t)row_bytes);
            else
                memcpy(d + seq[i] * row_bytes, s + i * row_bytes, (size_t)row_bytes);
        }
    }
    free(seq);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Review tokens                                                             */
/* ------------------------------------------------------------------------ */

/* Average-pool one batch element of a [T][H][W][C] tensor over disjoint
 * pt x ph x pw blocks, then unroll the pooled T' x H' x W' grid in RMS order
 * `order` (not flipped): out[j][c] for j = 0 .. T'H'W' - 1. */
int oracle_review_pool(const float *src, int64_t T, int64_t H, int64_t W, int64_t C, int pt,
                       int ph, int pw, int order, double *out)
{
    if (!src || !out || C <= 0 || pt <= 0 || ph <= 0 || pw <= 0) return ORACLE_EINVAL;
    if (T % pt || H % ph || W % pw) return ORACLE_EINVAL;
    int64_t Tp = T / pt, Hp = H / ph, Wp = W / pw, R = Tp * Hp * Wp;
    int64_t *seq = (int64_t *)malloc(sizeof(int64_t) * (size_t)R);
    double *pooled = (double *)calloc((size_t)(R * C), sizeof(double));
    if (!seq || !pooled) {
        free(seq);
        free(pooled);
        return ORACLE_ENOMEM;
    }
    double count = (double)pt * (double)ph * (double)pw;
    for (int64_t tq = 0; tq < Tp; ++tq)
        for (int64_t hq = 0; hq < Hp; ++hq)
            for (int64_t wq = 0; wq < Wp; ++wq) {
                double *acc = pooled + ((tq * Hp + hq) * Wp + wq) * C;
                for (int64_t t = tq * pt; t < (tq + 1) * pt; ++t)
                    for (int64_t h = hq * ph; h < (hq + 1) * ph; ++h)
                        for (int64_t w = wq * pw; w < (wq + 1) * pw; ++w) {
                            const float *row = src + ((t * H + h) * W + w) * C;
                            for (int64_t c = 0; c < C; ++c) acc[c] += (double)row[c];
                        }
                for (int64_t c = 0; c < C; ++c) acc[c] /= count;
            }
    int rc = oracle_rms_sequence(Tp, Hp, Wp, order, 0, seq);
    if (!rc)
        for (int64_t j = 0; j < R; ++j) memcpy(out + j * C, pooled + seq[j] * C, sizeof(double) * (size_t)C);
    free(seq);
    free(pooled);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* A tiny work queue over pthreads                                           */
/* ------------------------------------------------------------------------ */

/* A unit returns ORACLE_OK, or an error code (ORACLE_ENOMEM when it could not
 * allocate its scratch); run_units then returns the first error, so a failed
 * unit fails the whole call instead of leaving its outputs unwritten. */
typedef int (*unit_fn)(void *ctx, int64_t unit);
typedef struct {
    unit_fn fn;
    void *ctx;
    int64_t nunits;
    int64_t next;
    int failed;
    pthread_mutex_t lock;
} work_queue;

static void *worker(void *arg)
{
    work_queue *q = (work_queue *)arg;
    for (;;) {
        pthread_mutex_lock(&q->lock);
        int64_t u = q->next++;
        pthread_mutex_unlock(&q->lock);
        if (u >= q->nunits) break;
        int rc = q->fn(q->ctx, u);
        if (rc) {
            pthread_mutex_lock(&q->lock);
            if (!q->failed) q->failed = rc;
            q->next = q->nunits; /* no further units start */
            pthread_mutex_unlock(&q->lock);
        }
    }
    return NULL;
}

static int run_units(unit_fn fn, void *ctx, int64_t nunits, int nthreads)
{
    work_queue q;
    q.fn = fn;
    q.ctx = ctx;
    q.nunits = nunits;
    q.next = 0;
    q.failed = ORACLE_OK;
    pthread_mutex_init(&q.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 1024) nthreads = 1024;
    if ((int64_t)nthreads > nunits) nthreads = (int)(nunits > 0 ? nunits : 1);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 1; th && i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, worker, &q) == 0) ++started;
    worker(&q);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&q.lock);
    return q.failed;
}

/* ------------------------------------------------------------------------ */
/* Bidirectional Mamba2 scan                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float *x, *B, *C, *dt, *A, *D;
    int64_t batch, N, R;
    int nheads, P, S, G, head_lo, head_hi;
    const int64_t *seq;      /* scan order, N entries */
    const double *rx, *rB, *rdt; /* review tokens per batch: [b][R][nheads*P], [b][R][G*S], [b][R][nheads] */
    double *yf, *yb;         /* [b][N][nh][P] for the forward / backward direction */
} ssd_ctx;

/* One recurrence step on the P x S state of one head. */
static void ssd_step(double *h, int P, int S, double decay, double dt, const double *xv, const double *bv)
{
    for (int p = 0; p < P; ++p)
        for (int s = 0; s < S; ++s) h[p * S + s] = decay * h[p * S + s] + dt * xv[p] * bv[s];
}

static int ssd_unit(void *vctx, int64_t unit)
{
    ssd_ctx *c = (ssd_ctx *)vctx;
    int nh = c->head_hi - c->head_lo;
    int64_t b = unit / (2 * nh);
    int hl = (int)((unit / 2) % nh);
    int dir = (int)(unit % 2);
    int head = c->head_lo + hl;
    int g = head / (c->nheads / c->G); /* heads are split evenly over the B/C groups */
    int P = c->P, S = c->S;
    int64_t N = c->N, R = c->R;
    double A = (double)c->A[head], D = (double)c->D[head];
    double *h = (double *)calloc((size_t)P * S, sizeof(double));
    double *xv = (double *)malloc(sizeof(double) * P);
    double *bv = (double *)malloc(sizeof(double) * S);
    double *out = (dir == 0 ? c->yf : c->yb) + b * N * nh * P;
    if (!h || !xv || !bv) { free(h); free(xv); free(bv); return ORACLE_ENOMEM; }

    /* Review prefix: rev_o for the forward direction, its reversal for the
     * backward direction. Only the state is kept. */
    for (int64_t jj = 0; jj < R; ++jj) {
        int64_t j = dir == 0 ? jj : R - 1 - jj;
        const double *rx = c->rx + (b * R + j) * c->nheads * P + head * P;
        const double *rB = c->rB + (b * R + j) * c->G * S + g * S;
        double dt = c->rdt[(b * R + j) * c->nheads + head];
        ssd_step(h, P, S, exp(dt * A), dt, rx, rB);
    }
    /* Main sequence: seq_o forward, seq_o reversed backward. */
    for (int64_t ii = 0; ii < N; ++ii) {
        int64_t i = dir == 0 ? ii : N - 1 - ii;
        int64_t n = c->seq[i];
        const float *xr = c->x + ((b * N + n) * c->nheads + head) * P;
        const float *Br = c->B + ((b * N + n) * c->G + g) * S;
        const float *Cr = c->C + ((b * N + n) * c->G + g) * S;
        double dt = (double)c->dt[(b * N + n) * c->nheads + head];
        for (int p = 0; p < P; ++p) xv[p] = (double)xr[p];
        for (int s = 0; s < S; ++s) bv[s] = (double)Br[s];
        ssd_step(h, P, S, exp(dt * A), dt, xv, bv);
        double *yo = out + (n * nh + hl) * P;
        for (int p = 0; p < P; ++p) {
            double acc = 0.0;
            for (int s = 0; s < S; ++s) acc += h[p * S + s] * (double)Cr[s];
            yo[p] = acc + D * xv[p];
        }
    }
    free(h);
    free(xv);
    free(bv);
    return ORACLE_OK;
}

/* y[b][n][head - head_lo][p] for heads in [head_lo, head_hi).
 * x  [batch][T][H][W][nheads][P]      B, C [batch][T][H][W][G][S]
 * dt [batch][T][H][W][nheads] (> 0)    A, D [nheads]
 * pool_* all zero: no review tokens; otherwise they must divide T, H, W. */
int oracle_bissd(const float *x, const float *B, const float *C, const float *dt, const float *A,
                 const float *D, int64_t batch, int64_t T, int64_t H, int64_t W, int nheads, int P,
                 int S, int G, int order, int pool_t, int pool_h, int pool_w, int head_lo,
                 int head_hi, int nthreads, double *y)
{
    if (!x || !B || !C || !dt || !A || !D || !y) return ORACLE_EINVAL;
    if (batch <= 0 || T <= 0 || H <= 0 || W <= 0 || nheads <= 0 || P <= 0 || S <= 0 || G <= 0)
        return ORACLE_EINVAL;
    if (nheads % G || order < 0 || order > 4) return ORACLE_EINVAL;
    if (head_lo < 0 || head_hi > nheads || head_lo >= head_hi) return ORACLE_EINVAL;
    int pooled = pool_t || pool_h || pool_w;
    if (pooled && (pool_t <= 0 || pool_h <= 0 || pool_w <= 0 || T % pool_t || H % pool_h || W % pool_w))
        return ORACLE_EINVAL;
    int64_t N = T * H * W;
    int64_t R = pooled ? (T / pool_t) * (H / pool_h) * (W / pool_w) : 0;
    int nh = head_hi - head_lo;
    int rc = ORACLE_OK;

    int64_t *seq = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
    double *yb = (double *)malloc(sizeof(double) * (size_t)(batch * N * nh * P));
    double *rx = NULL, *rB = NULL, *rdt = NULL;
    if (!seq || !yb) { rc = ORACLE_ENOMEM; goto done; }
    rc = oracle_rms_sequence(T, H, W, order, 0, seq);
    if (rc) goto done;
    if (R > 0) {
        rx = (double *)malloc(sizeof(double) * (size_t)(batch * R * nheads * P));
        rB = (double *)malloc(sizeof(double) * (size_t)(batch * R * G * S));
        rdt = (double *)malloc(sizeof(double) * (size_t)(batch * R * nheads));
        if (!rx || !rB || !rdt) { rc = ORACLE_ENOMEM; goto done; }
        for (int64_t b = 0; b < batch && !rc; ++b) {
            rc = oracle_review_pool(x + b * N * nheads * P, T, H, W, (int64_t)nheads * P, pool_t, pool_h,
                                    pool_w, order, rx + b * R * nheads * P);
            if (!rc)
                rc = oracle_review_pool(B + b * N * G * S, T, H, W, (int64_t)G * S, pool_t, pool_h, pool_w,
                                        order, rB + b * R * G * S);
            if (!rc)
                rc = oracle_review_pool(dt + b * N * nheads, T, H, W, nheads, pool_t, pool_h, pool_w, order,
                                        rdt + b * R * nheads);
        }
        if (rc) goto done;
    }
    {
        ssd_ctx c;
        c.x = x; c.B = B; c.C = C; c.dt = dt; c.A = A; c.D = D;
        c.batch = batch; c.N = N; c.R = R;
        c.nheads = nheads; c.P = P; c.S = S; c.G = G; c.head_lo = head_lo; c.head_hi = head_hi;
        c.seq = seq; c.rx = rx; c.rB = rB; c.rdt = rdt;
        c.yf = y; c.yb = yb;
        rc = run_units(ssd_unit, &c, batch * nh * 2, nthreads);
        if (rc) goto done;
        int64_t total = batch * N * nh * P;
        for (int64_t e = 0; e < total; ++e) y[e] += yb[e];
    }
done:
    free(seq);
    free(yb);
    free(rx);
    free(rB);
    free(rdt);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Backward of the bidirectional Mamba2 scan                                 */
/* ------------------------------------------------------------------------ */
/* Gradients of the scan above for an upstream gradient dy of its output y
 * (the MA half of training the MATE block; the xllm-io review, section 三,
 * "训练配方", trains LinGen end to end). For one direction, over its sequence
 * z (review tokens, then the main tokens, as in the forward), with
 * a_u = exp(dt_u A), the forward recurrence
 *     h_u = a_u h_{u-1} + dt_u x_u B_u^T,   y_u = h_u C_u + D x_u
 * has the adjoint G_u = dL/dh_u, run from the end of z to its start:
 *     G_u = dy_u C_u^T + a_{u+1} G_{u+1}       (G after the last token is 0)
 * and the chain rule through each step gives, at position u,
 *     dx_u   += dt_u G_u B_u + D dy_u
 *     dB_u   += dt_u G_u^T x_u
 *     dC_u   += h_u^T dy_u
 *     ddt_u  += x_u^T G_u B_u + A a_u <h_{u-1}, G_u>
 *     dA     += dt_u a_u <h_{u-1}, G_u>
 *     dD     += x_u . dy_u
 * (<.,.> the sum of the elementwise product of two P x S matrices). dy is 0 at
 * review positions (their outputs are dropped), so pooled C gets no gradient;
 * the review tokens' dx, dB and ddt flow back through the average pooling: each
 * token of a pool block receives the block's gradient divided by the block's
 * token count. Both directions add into the same gradients.
 *
 * The states h_u that the adjoint needs are recomputed: the forward pass keeps
 * the state before every block of ORACLE_CKPT positions, and the backward pass
 * recomputes each block's states from its checkpoint before walking it
 * backwards. */
#define ORACLE_CKPT 256

typedef struct {
    const float *x, *B, *C, *dt, *A, *D, *dy;
    int64_t batch, N, R;
    int nheads, P, S, G, head_lo, head_hi;
    const int64_t *seq;            /* scan order, N entries */
    const double *rx, *rB, *rdt;   /* review tokens per batch: [b][R][nheads*P], [b][R][G*S], [b][R][nheads] */
    /* per (direction, batch, local head) results, written only by that unit; each array has one copy
     * per direction (index dir first), summed after all units have run */
    double *dx;                    /* [2][b][N][nh][P] */
    double *dBh, *dCh;             /* [2][b][nh][N][S]: this head's part of dB, dC */
    double *ddt;                   /* [2][b][N][nh] */
    double *drx, *drB, *drdt;      /* [2][b][nh][R][P], [2][b][nh][R][S], [2][b][nh][R]: review-token gradients */
    double *dA, *dD;               /* [2][b][nh] */
} ssd_bwd_ctx;

static int ssd_bwd_unit(void *vctx, int64_t unit)
{
    ssd_bwd_ctx *c = (ssd_bwd_ctx *)vctx;
    const int nh = c->head_hi - c->head_lo;
    const int64_t b = unit / (2 * nh);
    const int hl = (int)((unit / 2) % nh);
    const int dir = (int)(unit % 2);
    const int head = c->head_lo + hl;
    const int g = head / (c->nheads / c->G);
    const int P = c->P, S = c->S;
    const int64_t N = c->N, R = c->R, L = R + N, PS = (int64_t)P * S;
    const int64_t Rn = R > 0 ? R : 1, B = c->batch;
    /* this direction's copy of every result */
    double *dxo = c->dx + dir * B * N * nh * P, *dBo = c->dBh + dir * B * nh * N * S;
    double *dCo = c->dCh + dir * B * nh * N * S, *ddto = c->ddt + dir * B * N * nh;
    double *drxo = c->drx + dir * B * nh * Rn * P, *drBo = c->drB + dir * B * nh * Rn * S;
    double *drdto = c->drdt + dir * B * nh * Rn;
    const double A = (double)c->A[head], D = (double)c->D[head];
    const int64_t nblk = (L + ORACLE_CKPT - 1) / ORACLE_CKPT;

    double *ckpt = (double *)malloc(sizeof(double) * (size_t)(nblk * PS));   /* state before each block */
    double *hb = (double *)malloc(sizeof(double) * (size_t)(ORACLE_CKPT * PS)); /* states of one block */
    double *h = (double *)malloc(sizeof(double) * (size_t)PS);
    double *Gm = (double *)malloc(sizeof(double) * (size_t)PS);               /* G_u */
    double *carry = (double *)malloc(sizeof(double) * (size_t)PS);            /* a_{u+1} G_{u+1} */
    double *xv = (double *)malloc(sizeof(double) * (size_t)P), *dyv = (double *)malloc(sizeof(double) * (size_t)P);
    double *bv = (double *)malloc(sizeof(double) * (size_t)S), *cv = (double *)malloc(sizeof(double) * (size_t)S);
    double *gB = (double *)malloc(sizeof(double) * (size_t)P);
    if (!ckpt || !hb || !h || !Gm || !carry || !xv || !dyv || !bv || !cv || !gB) {
        free(ckpt); free(hb); free(h); free(Gm); free(carry); free(xv); free(dyv); free(bv); free(cv); free(gB);
        return ORACLE_ENOMEM;
    }
    double dA = 0.0, dD = 0.0;
    {
        /* Position u of this direction's sequence: its inputs, and where its gradients go. */
#define LOAD(u)                                                                                        \
    int64_t rj = -1, n = -1;                                                                           \
    double dtu;                                                                                        \
    if ((u) < R) {                                                                                     \
        rj = dir == 0 ? (u) : R - 1 - (u);                                                             \
        const double *rxp = c->rx + (b * R + rj) * c->nheads * P + (int64_t)head * P;                  \
        const double *rbp = c->rB + (b * R + rj) * c->G * S + (int64_t)g * S;                          \
        for (int p = 0; p < P; ++p) { xv[p] = rxp[p]; dyv[p] = 0.0; }                                  \
        for (int s = 0; s < S; ++s) { bv[s] = rbp[s]; cv[s] = 0.0; }                                   \
        dtu = c->rdt[(b * R + rj) * c->nheads + head];                                                 \
    } else {                                                                                           \
        const int64_t i = (u) - R;                                                                     \
        n = c->seq[dir == 0 ? i : N - 1 - i];                                                          \
        const float *xr = c->x + ((b * N + n) * c->nheads + head) * P;                                 \
        const float *dyr = c->dy + ((b * N + n) * c->nheads + head) * P;                               \
        const float *Br = c->B + ((b * N + n) * c->G + g) * S;                                         \
        const float *Cr = c->C + ((b * N + n) * c->G + g) * S;                                         \
        for (int p = 0; p < P; ++p) { xv[p] = (double)xr[p]; dyv[p] = (double)dyr[p]; }               \
        for (int s = 0; s < S; ++s) { bv[s] = (double)Br[s]; cv[s] = (double)Cr[s]; }                  \
        dtu = (double)c->dt[(b * N + n) * c->nheads + head];                                           \
    }
        /* Forward pass: the state before every block. */
        for (int64_t e = 0; e < PS; ++e) h[e] = 0.0;
        for (int64_t u = 0; u < L; ++u) {
            if (u % ORACLE_CKPT == 0) memcpy(ckpt + (u / ORACLE_CKPT) * PS, h, sizeof(double) * (size_t)PS);
            LOAD(u);
            (void)rj; (void)n;
            ssd_step(h, P, S, exp(dtu * A), dtu, xv, bv);
        }
        /* Backward pass, block by block from the end. */
        for (int64_t e = 0; e < PS; ++e) carry[e] = 0.0;
        for (int64_t k = nblk - 1; k >= 0; --k) {
            const int64_t u0 = k * ORACLE_CKPT, u1 = u0 + ORACLE_CKPT < L ? u0 + ORACLE_CKPT : L;
            memcpy(h, ckpt + k * PS, sizeof(double) * (size_t)PS);
            for (int64_t u = u0; u < u1; ++u) {
                LOAD(u);
                (void)rj; (void)n;
                ssd_step(h, P, S, exp(dtu * A), dtu, xv, bv);
                memcpy(hb + (u - u0) * PS, h, sizeof(double) * (size_t)PS);
            }
            for (int64_t u = u1 - 1; u >= u0; --u) {
                LOAD(u);
                const double au = exp(dtu * A);
                const double *hcur = hb + (u - u0) * PS;
                const double *hprev = u > u0 ? hb + (u - 1 - u0) * PS : ckpt + k * PS;
                double gh = 0.0, xgb = 0.0;
                for (int p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int s = 0; s < S; ++s) {
                        const double gv = dyv[p] * cv[s] + carry[p * S + s];
                        Gm[p * S + s] = gv;
                        acc += gv * bv[s];
                        gh += gv * hprev[p * S + s];
                    }
                    gB[p] = acc;
                    xgb += xv[p] * acc;
                }
                double *gx, *gbb, *gdt;
                if (rj >= 0) {
                    gx = drxo + ((b * nh + hl) * R + rj) * P;
                    gbb = drBo + ((b * nh + hl) * R + rj) * S;
                    gdt = drdto + (b * nh + hl) * R + rj;
                } else {
                    gx = dxo + ((b * N + n) * nh + hl) * P;
                    gbb = dBo + ((b * nh + hl) * N + n) * S;
                    gdt = ddto + (b * N + n) * nh + hl;
                    double *gc = dCo + ((b * nh + hl) * N + n) * S;
                    for (int s = 0; s < S; ++s) {
                        double acc = 0.0;
                        for (int p = 0; p < P; ++p) acc += hcur[p * S + s] * dyv[p];
                        gc[s] += acc;
                    }
                }
                for (int p = 0; p < P; ++p) gx[p] += dtu * gB[p] + D * dyv[p];
                for (int s = 0; s < S; ++s) {
                    double acc = 0.0;
                    for (int p = 0; p < P; ++p) acc += Gm[p * S + s] * xv[p];
                    gbb[s] += dtu * acc;
                }
                *gdt += xgb + A * au * gh;
                dA += dtu * au * gh;
                for (int p = 0; p < P; ++p) dD += xv[p] * dyv[p];
                for (int64_t e = 0; e < PS; ++e) carry[e] = au * Gm[e];
            }
        }
#undef LOAD
    }
    c->dA[(dir * B + b) * nh + hl] = dA;
    c->dD[(dir * B + b) * nh + hl] = dD;
    free(ckpt); free(hb); free(h); free(Gm); free(carry); free(xv); free(dyv); free(bv); free(cv); free(gB);
    return ORACLE_OK;
}

/* Gradients of oracle_bissd for the upstream gradient dy [batch][T][H][W][nheads][P]
 * (same arguments as oracle_bissd otherwise), for the heads in [head_lo, head_hi):
 *   dx  [batch][T][H][W][nh][P]      ddt [batch][T][H][W][nh]
 *   dB, dC [batch][T][H][W][G][S]   (summed over the heads in the range only)
 *   dA, dD [nh]                      (summed over the batch)
 * with nh = head_hi - head_lo. */
int oracle_bissd_backward(const float *x, const float *B, const float *C, const float *dt, const float *A,
                          const float *D, const float *dy, int64_t batch, int64_t T, int64_t H, int64_t W,
                          int nheads, int P, int S, int G, int order, int pool_t, int pool_h, int pool_w,
                          int head_lo, int head_hi, int nthreads, double *dx, double *dB, double *dC, double *ddt,
                          double *dA, double *dD)
{
    if (!x || !B || !C || !dt || !A || !D || !dy || !dx || !dB || !dC || !ddt || !dA || !dD) return ORACLE_EINVAL;
    if (batch <= 0 || T <= 0 || H <= 0 || W <= 0 || nheads <= 0 || P <= 0 || S <= 0 || G <= 0)
        return ORACLE_EINVAL;
    if (nheads % G || order < 0 || order > 4) return ORACLE_EINVAL;
    if (head_lo < 0 || head_hi > nheads || head_lo >= head_hi) return ORACLE_EINVAL;
    const int pooled = pool_t || pool_h || pool_w;
    if (pooled && (pool_t <= 0 || pool_h <= 0 || pool_w <= 0 || T % pool_t || H % pool_h || W % pool_w))
        return ORACLE_EINVAL;
    const int64_t N = T * H * W;
    const int64_t Tp = pooled ? T / pool_t : 0, Hp = pooled ? H / pool_h : 0, Wp = pooled ? W / pool_w : 0;
    const int64_t R = Tp * Hp * Wp;
    const int nh = head_hi - head_lo;
    int rc = ORACLE_OK;
    const int64_t Rn = R > 0 ? R : 1;
    int64_t *seq = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
    int64_t *rseq = (int64_t *)malloc(sizeof(int64_t) * (size_t)Rn);
    /* one copy per direction of every per-unit result */
    double *dx2 = (double *)calloc((size_t)(2 * batch * N * nh * P), sizeof(double));
    double *ddt2 = (double *)calloc((size_t)(2 * batch * N * nh), sizeof(double));
    double *dBh = (double *)calloc((size_t)(2 * batch * nh * N * S), sizeof(double));
    double *dCh = (double *)calloc((size_t)(2 * batch * nh * N * S), sizeof(double));
    double *drx = (double *)calloc((size_t)(2 * batch * nh * Rn * P), sizeof(double));
    double *drB = (double *)calloc((size_t)(2 * batch * nh * Rn * S), sizeof(double));
    double *drdt = (double *)calloc((size_t)(2 * batch * nh * Rn), sizeof(double));
    double *dAb = (double *)calloc((size_t)(2 * batch * nh), sizeof(double));
    double *dDb = (double *)calloc((size_t)(2 * batch * nh), sizeof(double));
    double *rx = NULL, *rB = NULL, *rdt = NULL;
    if (!seq || !rseq || !dx2 || !ddt2 || !dBh || !dCh || !drx || !drB || !drdt || !dAb || !dDb) {
        rc = ORACLE_ENOMEM;
        goto done;
    }
    rc = oracle_rms_sequence(T, H, W, order, 0, seq);
    if (rc) goto done;
    if (R > 0) {
        rc = oracle_rms_sequence(Tp, Hp, Wp, order, 0, rseq);
        if (rc) goto done;
        rx = (double *)malloc(sizeof(double) * (size_t)(batch * R * nheads * P));
        rB = (double *)malloc(sizeof(double) * (size_t)(batch * R * G * S));
        rdt = (double *)malloc(sizeof(double) * (size_t)(batch * R * nheads));
        if (!rx || !rB || !rdt) { rc = ORACLE_ENOMEM; goto done; }
        for (int64_t b = 0; b < batch && !rc; ++b) {
            rc = oracle_review_pool(x + b * N * nheads * P, T, H, W, (int64_t)nheads * P, pool_t, pool_h, pool_w,
                                    order, rx + b * R * nheads * P);
            if (!rc)
                rc = oracle_review_pool(B + b * N * G * S, T, H, W, (int64_t)G * S, pool_t, pool_h, pool_w, order,
                                        rB + b * R * G * S);
            if (!rc)
                rc = oracle_review_pool(dt + b * N * nheads, T, H, W, nheads, pool_t, pool_h, pool_w, order,
                                        rdt + b * R * nheads);
        }
        if (rc) goto done;
    }
    {
        ssd_bwd_ctx c;
        c.x = x; c.B = B; c.C = C; c.dt = dt; c.A = A; c.D = D; c.dy = dy;
        c.batch = batch; c.N = N; c.R = R;
        c.nheads = nheads; c.P = P; c.S = S; c.G = G; c.head_lo = head_lo; c.head_hi = head_hi;
        c.seq = seq; c.rx = rx; c.rB = rB; c.rdt = rdt;
        c.dx = dx2; c.dBh = dBh; c.dCh = dCh; c.ddt = ddt2; c.drx = drx; c.drB = drB; c.drdt = drdt;
        c.dA = dAb; c.dD = dDb;
        rc = run_units(ssd_bwd_unit, &c, batch * nh * 2, nthreads);
        if (rc) goto done;
    }
    /* The two directions summed (forward copy first). */
    {
        const int64_t nx = batch * N * nh * P, nd = batch * N * nh, ns = batch * nh * N * S;
        const int64_t nrx = batch * nh * Rn * P, nrb = batch * nh * Rn * S, nrd = batch * nh * Rn;
        for (int64_t e = 0; e < nx; ++e) dx[e] = dx2[e] + dx2[nx + e];
        for (int64_t e = 0; e < nd; ++e) ddt[e] = ddt2[e] + ddt2[nd + e];
        for (int64_t e = 0; e < ns; ++e) {
            dBh[e] += dBh[ns + e];
            dCh[e] += dCh[ns + e];
        }
        for (int64_t e = 0; e < nrx; ++e) drx[e] += drx[nrx + e];
        for (int64_t e = 0; e < nrb; ++e) drB[e] += drB[nrb + e];
        for (int64_t e = 0; e < nrd; ++e) drdt[e] += drdt[nrd + e];
        for (int64_t e = 0; e < batch * nh; ++e) {
            dAb[e] += dAb[batch * nh + e];
            dDb[e] += dDb[batch * nh + e];
        }
    }
    /* Review tokens back through the average pooling: every token of the block of review token j
     * (the pooled grid unrolled in the scan order) receives its gradient over the block's size. */
    if (R > 0) {
        const double inv = 1.0 / ((double)pool_t * pool_h * pool_w);
        for (int64_t b = 0; b < batch; ++b)
            for (int hl = 0; hl < nh; ++hl)
                for (int64_t j = 0; j < R; ++j) {
                    const int64_t pc = rseq[j];
                    const int64_t tq = pc / (Hp * Wp), hq = (pc / Wp) % Hp, wq = pc % Wp;
                    const double *gx = drx + ((b * nh + hl) * R + j) * P;
                    const double *gb = drB + ((b * nh + hl) * R + j) * S;
                    const double gd = drdt[(b * nh + hl) * R + j];
                    for (int64_t t = tq * pool_t; t < (tq + 1) * pool_t; ++t)
                        for (int64_t hh = hq * pool_h; hh < (hq + 1) * pool_h; ++hh)
                            for (int64_t w = wq * pool_w; w < (wq + 1) * pool_w; ++w) {
                                const int64_t n = (t * H + hh) * W + w;
                                for (int p = 0; p < P; ++p) dx[((b * N + n) * nh + hl) * P + p] += gx[p] * inv;
                                for (int s = 0; s < S; ++s) dBh[((b * nh + hl) * N + n) * S + s] += gb[s] * inv;
                                ddt[(b * N + n) * nh + hl] += gd * inv;
                            }
                }
    }
    /* dB and dC: each group's heads summed, in head order. */
    for (int64_t e = 0; e < batch * N * G * S; ++e) dB[e] = dC[e] = 0.0;
    for (int64_t b = 0; b < batch; ++b)
        for (int hl = 0; hl < nh; ++hl) {
            const int g = (head_lo + hl) / (nheads / G);
            for (int64_t n = 0; n < N; ++n)
                for (int s = 0; s < S; ++s) {
                    dB[((b * N + n) * G + g) * S + s] += dBh[((b * nh + hl) * N + n) * S + s];
                    dC[((b * N + n) * G + g) * S + s] += dCh[((b * nh + hl) * N + n) * S + s];
                }
        }
    for (int hl = 0; hl < nh; ++hl) {
        dA[hl] = dD[hl] = 0.0;
        for (int64_t b = 0; b < batch; ++b) {
            dA[hl] += dAb[b * nh + hl];
            dD[hl] += dDb[b * nh + hl];
        }
    }
done:
    free(seq); free(rseq); free(dx2); free(ddt2); free(dBh); free(dCh); free(drx); free(drB); free(drdt); free(dAb); free(dDb);
    free(rx); free(rB); free(rdt);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Bidirectional Mamba (selective scan), the MA branch of the ablation        */
/* ------------------------------------------------------------------------ */
/* The xllm-io review compares the MA branch built on Mamba with the one built
 * on Mamba2 (Table 2, row "Mamba", and the Mamba2 bullet under it). Mamba's
 * selective scan gives every channel c its own d_state states with their own
 * decay rates: A is a [channels][d_state] matrix and dt comes per channel,
 * where Mamba2 has one A and one dt per head. Per channel c and state s:
 *   h_u[c][s] = exp(dt_u[c] A[c][s]) h_{u-1}[c][s] + dt_u[c] x_u[c] B_u[s]
 *   y_u[c]    = sum_s C_u[s] h_u[c][s] + D[c] x_u[c]
 * The sequences, review tokens, flip and sum are those of the Mamba2 scan. */
typedef struct {
    const float *x, *B, *C, *dt, *A, *D;
    int64_t batch, N, R;
    int nch, S, ch_lo, ch_hi;
    const int64_t *seq;
    const double *rx, *rB, *rdt; /* review tokens per batch: [b][R][nch], [b][R][S], [b][R][nch] */
    double *yf, *yb;             /* [b][N][ch_hi - ch_lo] for the forward / backward direction */
} scan1_ctx;

static int scan1_unit(void *vctx, int64_t unit)
{
    scan1_ctx *c = (scan1_ctx *)vctx;
    int nc = c->ch_hi - c->ch_lo;
    int64_t b = unit / (2 * nc);
    int cl = (int)((unit / 2) % nc);
    int dir = (int)(unit % 2);
    int ch = c->ch_lo + cl;
    int S = c->S;
    int64_t N = c->N, R = c->R, nch = c->nch;
    const float *A = c->A + (int64_t)ch * S;
    double D = (double)c->D[ch];
    double *h = (double *)calloc((size_t)S, sizeof(double));
    double *out = (dir == 0 ? c->yf : c->yb) + b * N * nc;
    if (!h) return ORACLE_ENOMEM;
    for (int64_t jj = 0; jj < R; ++jj) {
        int64_t j = dir == 0 ? jj : R - 1 - jj;
        double xv = c->rx[(b * R + j) * nch + ch], dt = c->rdt[(b * R + j) * nch + ch];
        const double *Bv = c->rB + (b * R + j) * S;
        for (int s = 0; s < S; ++s) h[s] = exp(dt * (double)A[s]) * h[s] + dt * xv * Bv[s];
    }
    for (int64_t ii = 0; ii < N; ++ii) {
        int64_t i = dir == 0 ? ii : N - 1 - ii;
        int64_t n = c->seq[i];
        double xv = (double)c->x[(b * N + n) * nch + ch], dt = (double)c->dt[(b * N + n) * nch + ch];
        const float *Br = c->B + (b * N + n) * S, *Cr = c->C + (b * N + n) * S;
        double acc = 0.0;
        for (int s = 0; s < S; ++s) {
            h[s] = exp(dt * (double)A[s]) * h[s] + dt * xv * (double)Br[s];
            acc += (double)Cr[s] * h[s];
        }
        out[n * nc + cl] = acc + D * xv;
    }
    free(h);
    return ORACLE_OK;
}

/* y[b][n][c - ch_lo] for channels in [ch_lo, ch_hi).
 * x, dt [batch][T][H][W][nch] (dt > 0)   B, C [batch][T][H][W][S]
 * A [nch][S] (< 0)                        D [nch]
 * pool_* all zero: no review tokens; otherwise they must divide T, H, W. */
int oracle_biscan1(const float *x, const float *B, const float *C, const float *dt, const float *A,
                   const float *D, int64_t batch, int64_t T, int64_t H, int64_t W, int nch, int S,
                   int order, int pool_t, int pool_h, int pool_w, int ch_lo, int ch_hi, int nthreads,
                   double *y)
{
    if (!x || !B || !C || !dt || !A || !D || !y) return ORACLE_EINVAL;
    if (batch <= 0 || T <= 0 || H <= 0 || W <= 0 || nch <= 0 || S <= 0 || order < 0 || order > 4)
        return ORACLE_EINVAL;
    if (ch_lo < 0 || ch_hi > nch || ch_lo >= ch_hi) return ORACLE_EINVAL;
    int pooled = pool_t || pool_h || pool_w;
    if (pooled && (pool_t <= 0 || pool_h <= 0 || pool_w <= 0 || T % pool_t || H % pool_h || W % pool_w))
        return ORACLE_EINVAL;
    int64_t N = T * H * W;
    int64_t R = pooled ? (T / pool_t) * (H / pool_h) * (W / pool_w) : 0;
    int nc = ch_hi - ch_lo;
    int rc = ORACLE_OK;

    int64_t *seq = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
    double *yb = (double *)malloc(sizeof(double) * (size_t)(batch * N * nc));
    double *rx = NULL, *rB = NULL, *rdt = NULL;
    if (!seq || !yb) { rc = ORACLE_ENOMEM; goto done; }
    rc = oracle_rms_sequence(T, H, W, order, 0, seq);
    if (rc) goto done;
    if (R > 0) {
        rx = (double *)malloc(sizeof(double) * (size_t)(batch * R * nch));
        rB = (double *)malloc(sizeof(double) * (size_t)(batch * R * S));
        rdt = (double *)malloc(sizeof(double) * (size_t)(batch * R * nch));
        if (!rx || !rB || !rdt) { rc = ORACLE_ENOMEM; goto done; }
        for (int64_t b = 0; b < batch && !rc; ++b) {
            rc = oracle_review_pool(x + b * N * nch, T, H, W, nch, pool_t, pool_h, pool_w, order, rx + b * R * nch);
            if (!rc) rc = oracle_review_pool(B + b * N * S, T, H, W, S, pool_t, pool_h, pool_w, order, rB + b * R * S);
            if (!rc)
                rc = oracle_review_pool(dt + b * N * nch, T, H, W, nch, pool_t, pool_h, pool_w, order, rdt + b * R * nch);
        }
        if (rc) goto done;
    }
    {
        scan1_ctx c;
        c.x = x; c.B = B; c.C = C; c.dt = dt; c.A = A; c.D = D;
        c.batch = batch; c.N = N; c.R = R;
        c.nch = nch; c.S = S; c.ch_lo = ch_lo; c.ch_hi = ch_hi;
        c.seq = seq; c.rx = rx; c.rB = rB; c.rdt = rdt;
        c.yf = y; c.yb = yb;
        rc = run_units(scan1_unit, &c, batch * nc * 2, nthreads);
        if (rc) goto done;
        int64_t total = batch * N * nc;
        for (int64_t e = 0; e < total; ++e) y[e] += yb[e];
    }
done:
    free(seq);
    free(yb);
    free(rx);
    free(rB);
    free(rdt);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* TESA: attention inside shifted 3D windows                                  */
/* ------------------------------------------------------------------------ */

/* Region id of coordinate c along an axis with window w and shift s. */
static int64_t region_id(int64_t c, int64_t w, int64_t s) { return (c + w - s) / w; }

typedef struct {
    const float *q, *k, *v;
    int64_t batch, T, H, W, N;
    int nheads, d, head_lo, head_hi;
    int64_t wt, wh, ww, st, sh, sw;
    int64_t id0t, id0h, id0w; /* region id of coordinate 0 along each axis */
    int64_t nrt, nrh, nrw;    /* number of regions along each axis */
    const int64_t *regions;   /* region list (linear ids) or NULL for all */
    int64_t nregions;
    double scale;
    double *o;                /* [b][N][nh][d] */
} tesa_ctx;

static int tesa_unit(void *vctx, int64_t unit)
{
    tesa_ctx *c = (tesa_ctx *)vctx;
    int nh = c->head_hi - c->head_lo;
    int64_t r_idx = unit % c->nregions;
    int hl = (int)((unit / c->nregions) % nh);
    int64_t b = unit / (c->nregions * nh);
    int head = c->head_lo + hl;
    int64_t r = c->regions ? c->regions[r_idx] : r_idx;
    int64_t rw = r % c->nrw, rh = (r / c->nrw) % c->nrh, rt = r / (c->nrw * c->nrh);
    int64_t want_t = c->id0t + rt, want_h = c->id0h + rh, want_w = c->id0w + rw;
    int d = c->d;

    /* The region's tokens, in canonical order. */
    int64_t cap = c->wt * c->wh * c->ww, m = 0;
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    double *sc = (double *)malloc(sizeof(double) * (size_t)cap);
    if (!tok || !sc) { free(tok); free(sc); return ORACLE_ENOMEM; }
    for (int64_t t = 0; t < c->T; ++t) {
        if (region_id(t, c->wt, c->st) != want_t) continue;
        for (int64_t h = 0; h < c->H; ++h) {
            if (region_id(h, c->wh, c->sh) != want_h) continue;
            for (int64_t w = 0; w < c->W; ++w) {
                if (region_id(w, c->ww, c->sw) != want_w) continue;
                if (m < cap) tok[m] = (t * c->H + h) * c->W + w;
                ++m;
            }
        }
    }
    if (m > cap) m = cap; /* cannot happen: a region never exceeds the window */

    for (int64_t i = 0; i < m; ++i) {
        const float *qi = c->q + ((b * c->N + tok[i]) * c->nheads + head) * d;
        double mx = -INFINITY;
        for (int64_t j = 0; j < m; ++j) {
            const float *kj = c->k + ((b * c->N + tok[j]) * c->nheads + head) * d;
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += (double)qi[e] * (double)kj[e];
            sc[j] = c->scale * s;
            if (sc[j] > mx) mx = sc[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            sc[j] = exp(sc[j] - mx);
            l += sc[j];
        }
        double *oi = c->o + ((b * c->N + tok[i]) * nh + hl) * d;
        for (int e = 0; e < d; ++e) oi[e] = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            const float *vj = c->v + ((b * c->N + tok[j]) * c->nheads + head) * d;
            double pj = sc[j] / l;
            for (int e = 0; e < d; ++e) oi[e] += pj * (double)vj[e];
        }
    }
    free(tok);
    free(sc);
    return ORACLE_OK;
}

/* Gradients of TESA for an upstream gradient dO of the output. Inside each
 * region, with S = scale q k^T, P = softmax over each row of S and O = P v,
 * the chain rule through these steps gives
 *   dv = P^T dO,  dP = dO v^T,  dS_ij = P_ij (dP_ij - sum_l P_il dP_il),
 *   dq = scale dS k,  dk = scale dS^T q
 * (the backward pass of softmax attention; the pages train LinGen, the
 * xllm-io review, section 三, "训练配方", and this is TESA's part of it). */
int oracle_tesa_region_counts(int64_t T, int64_t H, int64_t W, int wt, int wh, int ww, int st, int sh,
                              int sw, int64_t *counts3);

typedef struct {
    tesa_ctx f;
    const float *dout;
    double *dq, *dk, *dv; /* [b][N][nh][d] */
} tesa_bwd_ctx;

static int tesa_bwd_unit(void *vctx, int64_t unit)
{
    tesa_bwd_ctx *cb = (tesa_bwd_ctx *)vctx;
    tesa_ctx *c = &cb->f;
    int nh = c->head_hi - c->head_lo;
    int64_t r_idx = unit % c->nregions;
    int hl = (int)((unit / c->nregions) % nh);
    int64_t b = unit / (c->nregions * nh);
    int head = c->head_lo + hl;
    int64_t r = c->regions ? c->regions[r_idx] : r_idx;
    int64_t rw = r % c->nrw, rh = (r / c->nrw) % c->nrh, rt = r / (c->nrw * c->nrh);
    int64_t want_t = c->id0t + rt, want_h = c->id0h + rh, want_w = c->id0w + rw;
    int d = c->d;

    int64_t cap = c->wt * c->wh * c->ww, m = 0;
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    if (!tok) return ORACLE_ENOMEM;
    for (int64_t t = 0; t < c->T; ++t) {
        if (region_id(t, c->wt, c->st) != want_t) continue;
        for (int64_t h = 0; h < c->H; ++h) {
            if (region_id(h, c->wh, c->sh) != want_h) continue;
            for (int64_t w = 0; w < c->W; ++w) {
                if (region_id(w, c->ww, c->sw) != want_w) continue;
                if (m < cap) tok[m] = (t * c->H + h) * c->W + w;
                ++m;
            }
        }
    }
    if (m > cap) m = cap;
    double *P = (double *)malloc(sizeof(double) * (size_t)(m * m));
    double *dP = (double *)malloc(sizeof(double) * (size_t)(m * m));
    if (!P || !dP) { free(tok); free(P); free(dP); return ORACLE_ENOMEM; }
#define ROW(ptr, i) ((ptr) + ((b * c->N + tok[i]) * c->nheads + head) * d)
#define OUT(ptr, i) ((ptr) + ((b * c->N + tok[i]) * nh + hl) * d)
    /* P: the softmax of each row of S. */
    for (int64_t i = 0; i < m; ++i) {
        double mx = -INFINITY, l = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += (double)ROW(c->q, i)[e] * (double)ROW(c->k, j)[e];
            P[i * m + j] = c->scale * s;
            if (P[i * m + j] > mx) mx = P[i * m + j];
        }
        for (int64_t j = 0; j < m; ++j) {
            P[i * m + j] = exp(P[i * m + j] - mx);
            l += P[i * m + j];
        }
        for (int64_t j = 0; j < m; ++j) P[i * m + j] /= l;
    }
    /* dP = dO v^T, then dS (kept in dP). */
    for (int64_t i = 0; i < m; ++i) {
        double rowdot = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += (double)ROW(cb->dout, i)[e] * (double)ROW(c->v, j)[e];
            dP[i * m + j] = s;
            rowdot += P[i * m + j] * s;
        }
        for (int64_t j = 0; j < m; ++j) dP[i * m + j] = P[i * m + j] * (dP[i * m + j] - rowdot);
    }
    for (int64_t i = 0; i < m; ++i) {
        double *dq = OUT(cb->dq, i), *dk = OUT(cb->dk, i), *dv = OUT(cb->dv, i);
        for (int e = 0; e < d; ++e) dq[e] = dk[e] = dv[e] = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            const double sij = dP[i * m + j], sji = dP[j * m + i], pji = P[j * m + i];
            for (int e = 0; e < d; ++e) {
                dq[e] += c->scale * sij * (double)ROW(c->k, j)[e];
                dk[e] += c->scale * sji * (double)ROW(c->q, j)[e];
                dv[e] += pji * (double)ROW(cb->dout, j)[e];
            }
        }
    }
#undef ROW
#undef OUT
    free(tok);
    free(P);
    free(dP);
    return ORACLE_OK;
}

/* dq, dk, dv [b][n][head - head_lo][e] for heads in [head_lo, head_hi), same
 * arguments as oracle_tesa plus dout [batch][T][H][W][nheads][d]. */
int oracle_tesa_backward(const float *q, const float *k, const float *v, const float *dout, int64_t batch,
                         int64_t T, int64_t H, int64_t W, int nheads, int d, int wt, int wh, int ww, int st,
                         int sh, int sw, double scale, int head_lo, int head_hi, const int64_t *regions,
                         int64_t nregions, int nthreads, double *dq, double *dk, double *dv)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || batch <= 0 || T <= 0 || H <= 0 || W <= 0 ||
        nheads <= 0 || d <= 0)
        return ORACLE_EINVAL;
    if (head_lo < 0 || head_hi > nheads || head_lo >= head_hi) return ORACLE_EINVAL;
    if (T % wt || H % wh || W % ww) return ORACLE_EINVAL;
    int64_t counts[3];
    int rc = oracle_tesa_region_counts(T, H, W, wt, wh, ww, st, sh, sw, counts);
    if (rc) return rc;
    int64_t total_regions = counts[0] * counts[1] * counts[2];
    if (regions) {
        for (int64_t i = 0; i < nregions; ++i)
            if (regions[i] < 0 || regions[i] >= total_regions) return ORACLE_EINVAL;
    } else {
        nregions = total_regions;
    }
    if (nregions <= 0) return ORACLE_OK;
    tesa_bwd_ctx cb;
    tesa_ctx *c = &cb.f;
    c->q = q; c->k = k; c->v = v;
    c->batch = batch; c->T = T; c->H = H; c->W = W; c->N = T * H * W;
    c->nheads = nheads; c->d = d; c->head_lo = head_lo; c->head_hi = head_hi;
    c->wt = wt; c->wh = wh; c->ww = ww; c->st = st; c->sh = sh; c->sw = sw;
    c->id0t = region_id(0, wt, st); c->id0h = region_id(0, wh, sh); c->id0w = region_id(0, ww, sw);
    c->nrt = counts[0]; c->nrh = counts[1]; c->nrw = counts[2];
    c->regions = regions; c->nregions = nregions;
    c->scale = scale > 0 ? scale : 1.0 / sqrt((double)d);
    c->o = NULL;
    cb.dout = dout; cb.dq = dq; cb.dk = dk; cb.dv = dv;
    return run_units(tesa_bwd_unit, &cb, batch * (int64_t)(head_hi - head_lo) * nregions, nthreads);
}

/* Number of regions along each axis (useful to build region lists). */
int oracle_tesa_region_counts(int64_t T, int64_t H, int64_t W, int wt, int wh, int ww, int st, int sh,
                              int sw, int64_t *counts3)
{
    if (!counts3 || wt <= 0 || wh <= 0 || ww <= 0) return ORACLE_EINVAL;
    if (st < 0 || st >= wt || sh < 0 || sh >= wh || sw < 0 || sw >= ww) return ORACLE_EINVAL;
    counts3[0] = region_id(T - 1, wt, st) - region_id(0, wt, st) + 1;
    counts3[1] = region_id(H - 1, wh, sh) - region_id(0, wh, sh) + 1;
    counts3[2] = region_id(W - 1, ww, sw) - region_id(0, ww, sw) + 1;
    return ORACLE_OK;
}

/* o[b][n][head - head_lo][e] for heads in [head_lo, head_hi).
 * q, k, v [batch][T][H][W][nheads][d]. regions: NULL for every region, else a
 * list of linear region ids (rt * nrh + rh) * nrw + rw; only tokens of the
 * listed regions are written. scale <= 0 selects 1/sqrt(d). */
int oracle_tesa(const float *q, const float *k, const float *v, int64_t batch, int64_t T, int64_t H,
                int64_t W, int nheads, int d, int wt, int wh, int ww, int st, int sh, int sw, double scale,
                int head_lo, int head_hi, const int64_t *regions, int64_t nregions, int nthreads, double *o)
{
    if (!q || !k || !v || !o || batch <= 0 || T <= 0 || H <= 0 || W <= 0 || nheads <= 0 || d <= 0)
        return ORACLE_EINVAL;
    if (head_lo < 0 || head_hi > nheads || head_lo >= head_hi) return ORACLE_EINVAL;
    if (T % wt || H % wh || W % ww) return ORACLE_EINVAL;
    int64_t counts[3];
    int rc = oracle_tesa_region_counts(T, H, W, wt, wh, ww, st, sh, sw, counts);
    if (rc) return rc;
    int64_t total_regions = counts[0] * counts[1] * counts[2];
    if (regions) {
        for (int64_t i = 0; i < nregions; ++i)
            if (regions[i] < 0 || regions[i] >= total_regions) return ORACLE_EINVAL;
    } else {
        nregions = total_regions;
    }
    if (nregions <= 0) return ORACLE_OK;
    tesa_ctx c;
    c.q = q; c.k = k; c.v = v;
    c.batch = batch; c.T = T; c.H = H; c.W = W; c.N = T * H * W;
    c.nheads = nheads; c.d = d; c.head_lo = head_lo; c.head_hi = head_hi;
    c.wt = wt; c.wh = wh; c.ww = ww; c.st = st; c.sh = sh; c.sw = sw;
    c.id0t = region_id(0, wt, st); c.id0h = region_id(0, wh, sh); c.id0w = region_id(0, ww, sw);
    c.nrt = counts[0]; c.nrh = counts[1]; c.nrw = counts[2];
    c.regions = regions; c.nregions = nregions;
    c.scale = scale > 0 ? scale : 1.0 / sqrt((double)d);
    c.o = o;
    return run_units(tesa_unit, &c, batch * (int64_t)(head_hi - head_lo) * nregions, nthreads);
}
