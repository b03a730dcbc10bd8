// Backward of the bidirectional Mamba2 scan: dx, dB, dC, ddt, dA, dD for an
// upstream gradient dy of y (fp32 arithmetic, chunked).
//
// Chunks of Q tokens (Q = 64, or 32 for wide heads), with cs_t the inclusive
// and ce_t = cs_t - dt_t A the exclusive cumulative sum of dt A inside the
// chunk and tot = cs_{Q-1}. The forward pass is the sum over both directions of
//   y_t = sum_u (C_t . B_u) L_tu x_u + exp(cs_t) Hf C_t + exp(tot - ce_t) Hb C_t + 2 D x_t
// with L_tu = dt_u exp(cs_t - cs_u) below the diagonal, dt_u exp(ce_u - ce_t)
// above it and 2 dt_t on it; Hf (Hb) is the state entering the chunk from the
// left (right). Its adjoint states, Gf (gradient of the forward state leaving
// the chunk to the right, from the chunks after it) and Gb (of the backward
// state leaving it to the left, from the chunks before it), follow the same
// chunk recurrence with dy_t C_t^T in place of dt_u x_u B_u^T and the roles of
// the two directions exchanged:
//   Gf(c-1) = exp(tot_c) Gf(c) + sum_t exp(cs_t) dy_t C_t^T,
//   Gb(c+1) = exp(tot_c) Gb(c) + sum_t exp(tot - ce_t) dy_t C_t^T.
// Per chunk, with M = (C B^T) o L, DX_tu = dy_t . x_u and Z = DX o L:
//   dx_u = sum_t M_tu dy_t + dt_u exp(tot - cs_u) Gf B_u + dt_u exp(ce_u) Gb B_u + 2 D dy_u
//   dC_t = sum_u Z_tu B_u + exp(cs_t) Hf^T dy_t + exp(tot - ce_t) Hb^T dy_t        (summed over heads)
//   dB_u = sum_t Z_tu C_t + dt_u exp(tot - cs_u) Gf^T x_u + dt_u exp(ce_u) Gb^T x_u (summed over heads)
// dt enters twice: as the factor dt_u of L (x_k . (dx_k - 2 D dy_k) / dt_k) and
// through the decays: a pair (t, u) of the forward direction decays by the dt A
// of the positions u < k <= t, one of the backward direction by those of
// t <= k < u, so ddt_k gets A times the sum of W_tu = M_tu DX_tu over the pairs
// that span k, and dA the sum over k of dt_k times that. Those sums are formed
// locally, chunk by chunk: the pairs inside the chunk (prefix sums of the
// strict row and column sums of W), pairs with one end in the chunk and one
// outside (per-token products with the states), and pairs that span the whole
// chunk (exp(tot) <Hf, Gf> and exp(tot) <Hb, Gb>), so no sum runs over the
// whole sequence. Review tokens (whose outputs are dropped, dy = 0) receive the
// adjoints of the initial states, and their gradients flow back through the
// average pooling to the tokens of their pool blocks.
#include "common.hpp"
#include "launch.hpp"
#include "ssd_chunks.hpp"
#include "ssd_common.hpp"
#include "timing.hpp"

namespace mate {

namespace {

using ssd::k_cb;
using ssd::k_chunk_states;
using ssd::k_pool;
using ssd::k_prep_dt;
using ssd::k_state_pass;

constexpr int NTB = 256;  // threads per workgroup
constexpr int SL = 32;    // width of the state slices staged in LDS

// Per-token values of one chunk and head: dt, cs, ce and the two state weights
// ef = dt exp(tot - cs), eb = dt exp(ce).
struct TokLds {
    float *dt, *cs, *ce, *ef, *eb;
};

__device__ __forceinline__ void load_tokens(const TokLds &tk, const float *dtT, const float *csT, size_t row, int Q,
                                            float a)
{
    const float tot = csT[row + Q - 1];
    for (int u = threadIdx.x; u < Q; u += NTB) {
        const float d = dtT[row + u], cs = csT[row + u], ce = cs - d * a;
        tk.dt[u] = d;
        tk.cs[u] = cs;
        tk.ce[u] = ce;
        tk.ef[u] = d * __expf(tot - cs);
        tk.eb[u] = d * __expf(ce);
    }
}

// L_tu (the bidirectional decay times dt_u, 2 dt on the diagonal).
__device__ __forceinline__ float ldt(const TokLds &tk, int t, int u)
{
    if (u < t) return tk.dt[u] * __expf(tk.cs[t] - tk.cs[u]);
    if (u > t) return tk.dt[u] * __expf(tk.ce[u] - tk.ce[t]);
    return 2.f * tk.dt[t];
}

// Rows [Q][ld] of a token tensor (cols channels of head/group `hd` of `nh`), zero past the end.
template <typename E>
__device__ __forceinline__ void load_rows(float *dst, int ld, const E *src, int cols, int nh, int hd, uint32_t c, int Q,
                                          uint32_t N, size_t b, int order, uint32_t T, uint32_t H, uint32_t W)
{
    for (int k = threadIdx.x; k < Q * cols; k += NTB) {
        const int u = k / cols, p = k - u * cols;
        const uint32_t i = c * Q + u;
        float v = 0.f;
        if (i < N) v = elem<E>::load(src + ((b * N + rms_index32(i, order, T, H, W)) * nh + hd) * cols + p);
        dst[u * ld + p] = v;
    }
}

// Sum over the lanes of one segment of `seg` consecutive lanes (seg a power of two, <= 64).
__device__ __forceinline__ float seg_sum(float v, int seg)
{
    for (int off = seg >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Review-token index of canonical token n (its pool block, unrolled in the scan order).
__device__ __forceinline__ uint32_t review_of(uint32_t n, const int *rinv, uint32_t H, uint32_t W, int pt, int ph,
                                              int pw)
{
    const uint32_t t = n / (H * W), h = (n / W) % H, w = n % W;
    const uint32_t Hp = H / ph, Wp = W / pw;
    return (uint32_t)rinv[((t / pt) * Hp + h / ph) * Wp + w / pw];
}

// ---------------------------------------------------------------------------
// rinv[pooled canonical index] = review index j (the pooled grid in RMS order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_review_index(int *__restrict__ rinv, uint32_t R, int order, uint32_t Tp,
                                                      uint32_t Hp, uint32_t Wp)
{
    const uint32_t j = blockIdx.x * 256 + threadIdx.x;
    if (j < R) rinv[rms_index32(j, order, Tp, Hp, Wp)] = (int)j;
}

// ---------------------------------------------------------------------------
// Gradients of the review tokens of one (batch, head). Forward direction: the
// adjoint of the state the review tokens leave to the main sequence is Gf0; a
// review token r reaches it with decay df_r = exp(sum_{j > r} dt_j A). Backward
// direction (review tokens taken in reverse order): Gb0 and db_r = exp(sum_{j < r}
// dt_j A). dy is 0 on review tokens, so each token's pairs are with main tokens
// only and the pairs spanning r are those whose review end lies before r in
// that direction. grid (batch * nheads), 256 threads; P <= 64, S <= 128.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NTB) void k_review_grads(const float *__restrict__ rx, const float *__restrict__ rB,
                                                      const float *__restrict__ rdt, const float *__restrict__ A,
                                                      const float *__restrict__ Gf0, const float *__restrict__ Gb0,
                                                      float *__restrict__ drx, float *__restrict__ drB,
                                                      float *__restrict__ drdt, float *__restrict__ pAr, int nheads,
                                                      int P, int S, int G, int R)
{
    extern __shared__ float sm[];
    const int PS = P * S;
    float *gf = sm, *gb = gf + PS;             // adjoint states [P][S]
    float *xs = gb + PS, *bs = xs + P;         // the token's x and B
    float *decf = bs + S, *decb = decf + R;    // decays to the review end, per direction
    float *cfr = decb + R, *cbr = cfr + R;     // per-token pair sums (dt x . dx-part)
    float *red = cbr + R;                      // [2][NTB] partial sums
    const int bh = blockIdx.x, b = bh / nheads, h = bh % nheads, g = h / (nheads / G);
    const float a = A[h];
    for (int e = threadIdx.x; e < PS; e += NTB) {
        gf[e] = Gf0[(size_t)bh * PS + e];
        gb[e] = Gb0[(size_t)bh * PS + e];
    }
    if (threadIdx.x == 0) {
        float run = 1.f;
        for (int r = R - 1; r >= 0; --r) {
            decf[r] = run;
            run *= __expf(rdt[((size_t)b * R + r) * nheads + h] * a);
        }
        run = 1.f;
        for (int r = 0; r < R; ++r) {
            decb[r] = run;
            run *= __expf(rdt[((size_t)b * R + r) * nheads + h] * a);
        }
    }
    __syncthreads();
    // thread layout: for G x B (P outputs), 4 threads per p split S; for G^T x (S outputs), 2 threads per s split P
    const int tp = threadIdx.x >> 2, tq = threadIdx.x & 3;
    const int ts = threadIdx.x >> 1, tr = threadIdx.x & 1;
    for (int r = 0; r < R; ++r) {
        const float d = rdt[((size_t)b * R + r) * nheads + h];
        for (int p = threadIdx.x; p < P; p += NTB) xs[p] = rx[((size_t)b * R + r) * nheads * P + (size_t)h * P + p];
        for (int s = threadIdx.x; s < S; s += NTB) bs[s] = rB[((size_t)b * R + r) * G * S + (size_t)g * S + s];
        __syncthreads();
        // G B_r (P values) for both directions
        float pf = 0.f, pb = 0.f;
        if (tp < P)
            for (int s = tq; s < S; s += 4) {
                pf += gf[tp * S + s] * bs[s];
                pb += gb[tp * S + s] * bs[s];
            }
        pf = seg_sum(pf, 4);
        pb = seg_sum(pb, 4);
        // dx = dt dec (G B); the explicit dt part x . (dec G B)
        float xf = 0.f, xb = 0.f;
        if (tp < P && tq == 0) {
            const float vf = decf[r] * pf, vb = decb[r] * pb;
            drx[(((size_t)b * R + r) * nheads + h) * P + tp] = d * (vf + vb);
            xf = xs[tp] * vf;
            xb = xs[tp] * vb;
        }
        // G^T x_r (S values)
        float qf = 0.f, qb = 0.f;
        if (ts < S)
            for (int p = tr; p < P; p += 2) {
                qf += gf[p * S + ts] * xs[p];
                qb += gb[p * S + ts] * xs[p];
            }
        qf = seg_sum(qf, 2);
        qb = seg_sum(qb, 2);
        if (ts < S && tr == 0)
            drB[(((size_t)b * R + r) * nheads + h) * S + ts] = d * (decf[r] * qf + decb[r] * qb);
        // block sums of the explicit parts
        red[threadIdx.x] = xf;
        red[NTB + threadIdx.x] = xb;
        __syncthreads();
        if (threadIdx.x == 0) {
            float ef = 0.f, eb = 0.f;
            for (int k = 0; k < NTB; ++k) {
                ef += red[k];
                eb += red[NTB + k];
            }
            drdt[((size_t)b * R + r) * nheads + h] = ef + eb;  // explicit part; decay part added below
            cfr[r] = d * ef;
            cbr[r] = d * eb;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        // spans: forward pairs spanning r have their review end u < r; backward pairs u > r
        float below = 0.f, dA = 0.f;
        for (int r = 0; r < R; ++r) {
            float *o = drdt + ((size_t)b * R + r) * nheads + h;
            *o += a * below;
            dA += rdt[((size_t)b * R + r) * nheads + h] * below;
            below += cfr[r];
        }
        float above = 0.f;
        for (int r = R - 1; r >= 0; --r) {
            float *o = drdt + ((size_t)b * R + r) * nheads + h;
            *o += a * above;
            dA += rdt[((size_t)b * R + r) * nheads + h] * above;
            above += cbr[r];
        }
        pAr[bh] = dA;
    }
}

// drBg[b][r][g][s] = sum over the heads of group g of drB[b][r][h][s]. grid (R, batch), 256 threads.
__global__ __launch_bounds__(256) void k_review_group(const float *__restrict__ drB, float *__restrict__ drBg,
                                                      int nheads, int S, int G)
{
    const int r = blockIdx.x, b = blockIdx.y, R = gridDim.x;
    const int hpg = nheads / G;
    for (int e = threadIdx.x; e < G * S; e += 256) {
        const int g = e / S, s = e - g * S;
        float acc = 0.f;
        for (int k = 0; k < hpg; ++k) acc += drB[(((size_t)b * R + r) * nheads + g * hpg + k) * S + s];
        drBg[(((size_t)b * R + r) * G + g) * S + s] = acc;
    }
}

// ---------------------------------------------------------------------------
// dx of one chunk and head, with the per-token sums the dt gradient needs:
//   expl_u = x_u . (dx_u - 2 D dy_u) / dt_u,  cf_u = x_u . (dt_u exp(tot - cs_u) Gf B_u),
//   cb_u = x_u . (dt_u exp(ce_u) Gb B_u).
// grid (nch, nheads, batch), 256 threads; P in {16, 32, 64}.
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(NTB) void k_bwd_dx(const E *__restrict__ x, const E *__restrict__ dy,
                                                const E *__restrict__ Bm, const float *__restrict__ CB,
                                                const float *__restrict__ dtT, const float *__restrict__ csT,
                                                const float *__restrict__ A, const float *__restrict__ Dv,
                                                const float *__restrict__ Gf, const float *__restrict__ Gb,
                                                const float *__restrict__ drx, const int *__restrict__ rinv,
                                                E *__restrict__ dx, float *__restrict__ expl, float *__restrict__ cfo,
                                                float *__restrict__ cbo, int nheads, int P, int S, int G, uint32_t N,
                                                uint32_t Lpad, int Q, int order, uint32_t T, uint32_t H, uint32_t W,
                                                int pt, int ph, int pw, uint32_t R)
{
    extern __shared__ float sm[];
    const int LP = P + 1, LS = S + 1, LQ = Q + 1;
    float *sM = sm;                  // [Q][Q+1]  M_tu = CB_tu L_tu
    float *sY = sM + Q * LQ;         // [Q][P+1]  dy
    float *sX = sY + Q * LP;         // [Q][P+1]  x
    float *sB = sX + Q * LP;         // [Q][S+1]  B
    float *sGf = sB + Q * LS;        // [P][SL+1] slice of Gf
    float *sGb = sGf + P * (SL + 1); // [P][SL+1] slice of Gb
    float *tkm = sGb + P * (SL + 1);
    const TokLds tk{tkm, tkm + Q, tkm + 2 * Q, tkm + 3 * Q, tkm + 4 * Q};
    float *s_expl = tkm + 5 * Q, *s_cf = s_expl + Q, *s_cb = s_cf + Q;
    const uint32_t c = blockIdx.x, nch = gridDim.x;
    const int h = blockIdx.y, g = h / (nheads / G);
    const size_t b = blockIdx.z;
    const size_t row = (b * nheads + h) * Lpad + (size_t)c * Q;
    const float a = A[h];
    load_tokens(tk, dtT, csT, row, Q, a);
    load_rows(sY, LP, dy, P, nheads, h, c, Q, N, b, order, T, H, W);
    load_rows(sX, LP, x, P, nheads, h, c, Q, N, b, order, T, H, W);
    load_rows(sB, LS, Bm, S, G, g, c, Q, N, b, order, T, H, W);
    __syncthreads();
    const float *cb = CB + ((b * G + g) * nch + c) * (size_t)Q * Q;
    for (int k = threadIdx.x; k < Q * Q; k += NTB) {
        const int t = k / Q, u = k - t * Q;
        sM[t * LQ + u] = cb[k] * ldt(tk, t, u);
    }
    __syncthreads();
    // outputs (u, p), e = tid + NTB k: u = e / P, p = e % P (a segment of P lanes shares u)
    constexpr int MAXI = 64 * 64 / NTB;
    const int items = (Q * P + NTB - 1) / NTB;
    float acc[MAXI], af[MAXI], ab[MAXI];
#pragma unroll
    for (int k = 0; k < MAXI; ++k) acc[k] = af[k] = ab[k] = 0.f;
#pragma unroll
    for (int k = 0; k < MAXI; ++k) {
        const int e = threadIdx.x + NTB * k;
        if (k < items && e < Q * P) {
            const int u = e / P, p = e - u * P;
            float s_ = 0.f;
            for (int t = 0; t < Q; ++t) s_ += sM[t * LQ + u] * sY[t * LP + p];
            acc[k] = s_;
        }
    }
    const size_t PS = (size_t)P * S;
    const float *gf = Gf + ((b * nheads + h) * nch + c) * PS;
    const float *gb = Gb + ((b * nheads + h) * nch + c) * PS;
    for (int s0 = 0; s0 < S; s0 += SL) {
        __syncthreads();
        for (int k = threadIdx.x; k < P * SL; k += NTB) {
            const int p = k / SL, s = k - p * SL;
            const bool ok = s0 + s < S;
            sGf[p * (SL + 1) + s] = ok ? gf[p * S + s0 + s] : 0.f;
            sGb[p * (SL + 1) + s] = ok ? gb[p * S + s0 + s] : 0.f;
        }
        __syncthreads();
        const int sn = min(SL, S - s0);
#pragma unroll
        for (int k = 0; k < MAXI; ++k) {
            const int e = threadIdx.x + NTB * k;
            if (k < items && e < Q * P) {
                const int u = e / P, p = e - u * P;
                float vf = 0.f, vb = 0.f;
                for (int s = 0; s < sn; ++s) {
                    const float bv = sB[u * LS + s0 + s];
                    vf += sGf[p * (SL + 1) + s] * bv;
                    vb += sGb[p * (SL + 1) + s] * bv;
                }
                af[k] += vf;
                ab[k] += vb;
            }
        }
    }
    const float twoD = 2.f * Dv[h];
    const float inv_cnt = R > 0 ? 1.f / (float)(pt * ph * pw) : 0.f;
#pragma unroll
    for (int k = 0; k < MAXI; ++k) {
        const int e = threadIdx.x + NTB * k;
        if (k < items) {
            const bool ok = e < Q * P;
            const int u = ok ? e / P : 0, p = ok ? e - u * P : 0;
            const uint32_t i = c * Q + u;
            const float sf = tk.ef[u] * af[k], sb = tk.eb[u] * ab[k];
            const float scan = acc[k] + sf + sb;
            const float xv = sX[u * LP + p];
            const float d = tk.dt[u];
            float pe = ok && d > 0.f ? xv * scan / d : 0.f, pf = ok ? xv * sf : 0.f, pb = ok ? xv * sb : 0.f;
            pe = seg_sum(pe, P);
            pf = seg_sum(pf, P);
            pb = seg_sum(pb, P);
            if (ok && p == 0) {
                s_expl[u] = pe;
                s_cf[u] = pf;
                s_cb[u] = pb;
            }
            if (ok && i < N) {
                const uint32_t n = rms_index32(i, order, T, H, W);
                float v = scan + twoD * sY[u * LP + p];
                if (R > 0) v += drx[((b * R + review_of(n, rinv, H, W, pt, ph, pw)) * nheads + h) * P + p] * inv_cnt;
                elem<E>::store(dx + ((b * N + n) * nheads + h) * P + p, v);
            }
        }
    }
    __syncthreads();
    for (int u = threadIdx.x; u < Q; u += NTB) {
        expl[row + u] = s_expl[u];
        cfo[row + u] = s_cf[u];
        cbo[row + u] = s_cb[u];
    }
}

// ---------------------------------------------------------------------------
// dB and dC of one chunk and group (the heads of the group in turn, summed in
// registers), with the per-head token sums rf_t = exp(cs_t) C_t . (Hf^T dy_t)
// and rb_t = exp(tot - ce_t) C_t . (Hb^T dy_t). Outputs (t, s) are taken in
// slices of SL state columns: item k of a thread is slice k / IPS, token
// tid / SL + (NTB / SL) (k % IPS), column tid % SL, so every thread works on
// every slice. grid (nch, G, batch), 256 threads; Q <= 64, S <= 128.
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(NTB) void k_bwd_dbdc(const E *__restrict__ x, const E *__restrict__ dy,
                                                  const E *__restrict__ Bm, const E *__restrict__ Cm,
                                                  const float *__restrict__ dtT, const float *__restrict__ csT,
                                                  const float *__restrict__ A, const float *__restrict__ Hf,
                                                  const float *__restrict__ Hb, const float *__restrict__ Gf,
                                                  const float *__restrict__ Gb, const float *__restrict__ drBg,
                                                  const int *__restrict__ rinv, E *__restrict__ dB,
                                                  E *__restrict__ dC, float *__restrict__ rfo, float *__restrict__ rbo,
                                                  int nheads, int P, int S, int G, uint32_t N, uint32_t Lpad, int Q,
                                                  int order, uint32_t T, uint32_t H, uint32_t W, int pt, int ph, int pw,
                                                  uint32_t R)
{
    extern __shared__ float sm[];
    const int LP = P + 1, LS = S + 1, LQ = Q + 1, LL = SL + 1;
    float *sB = sm;                   // [Q][S+1]
    float *sC = sB + Q * LS;          // [Q][S+1]
    float *sX = sC + Q * LS;          // [Q][P+1]
    float *sY = sX + Q * LP;          // [Q][P+1]
    float *sZ = sY + Q * LP;          // [Q][Q+1]  Z_tu = (dy_t . x_u) L_tu
    float *sHf = sZ + Q * LQ;         // [P][SL+1] slices of Hf, Hb, Gf, Gb
    float *sHb = sHf + P * LL;
    float *sGf = sHb + P * LL;
    float *sGb = sGf + P * LL;
    float *tkm = sGb + P * LL;
    const TokLds tk{tkm, tkm + Q, tkm + 2 * Q, tkm + 3 * Q, tkm + 4 * Q};
    const uint32_t c = blockIdx.x, nch = gridDim.x;
    const int g = blockIdx.y, hpg = nheads / G;
    const size_t b = blockIdx.z;
    load_rows(sB, LS, Bm, S, G, g, c, Q, N, b, order, T, H, W);
    load_rows(sC, LS, Cm, S, G, g, c, Q, N, b, order, T, H, W);
    constexpr int IPS = 64 * SL / NTB;       // items per slice (Q = 64 at most)
    constexpr int MAXI = IPS * (128 / SL);   // S = 128 at most
    const int nsl = (S + SL - 1) / SL;
    const int tcol = threadIdx.x % SL, trow = threadIdx.x / SL;  // item: token trow + (NTB / SL) k', column tcol
    float accB[MAXI], accC[MAXI];
#pragma unroll
    for (int k = 0; k < MAXI; ++k) accB[k] = accC[k] = 0.f;
    const size_t PS = (size_t)P * S;
    for (int hk = 0; hk < hpg; ++hk) {
        const int h = g * hpg + hk;
        const float a = A[h];
        const size_t row = (b * nheads + h) * Lpad + (size_t)c * Q;
        __syncthreads();  // the previous head's reads of sX, sY, sZ and the tokens are done
        load_tokens(tk, dtT, csT, row, Q, a);
        load_rows(sX, LP, x, P, nheads, h, c, Q, N, b, order, T, H, W);
        load_rows(sY, LP, dy, P, nheads, h, c, Q, N, b, order, T, H, W);
        __syncthreads();
        for (int k = threadIdx.x; k < Q * Q; k += NTB) {
            const int t = k / Q, u = k - t * Q;
            float s_ = 0.f;
            for (int p = 0; p < P; ++p) s_ += sY[t * LP + p] * sX[u * LP + p];
            sZ[t * LQ + u] = s_ * ldt(tk, t, u);
        }
        const size_t so = ((b * nheads + h) * nch + c) * PS;
        float rf[IPS], rb[IPS];
#pragma unroll
        for (int k = 0; k < IPS; ++k) rf[k] = rb[k] = 0.f;
        for (int sl = 0; sl < nsl; ++sl) {
            const int s0 = sl * SL;
            __syncthreads();  // sZ complete; the previous slice's reads are done
            for (int k = threadIdx.x; k < P * SL; k += NTB) {
                const int p = k / SL, s = k - p * SL;
                const bool ok = s0 + s < S;
                const size_t o = so + (size_t)p * S + s0 + s;
                sHf[p * LL + s] = ok ? Hf[o] : 0.f;
                sHb[p * LL + s] = ok ? Hb[o] : 0.f;
                sGf[p * LL + s] = ok ? Gf[o] : 0.f;
                sGb[p * LL + s] = ok ? Gb[o] : 0.f;
            }
            __syncthreads();
            const int s = s0 + tcol;
#pragma unroll
            for (int k2 = 0; k2 < IPS; ++k2) {
                const int t = trow + (NTB / SL) * k2;  // also the token u of dB
                if (t < Q && s < S) {
                    float zc = 0.f, zb = 0.f;
                    for (int u = 0; u < Q; ++u) {
                        zc += sZ[t * LQ + u] * sB[u * LS + s];  // dC_t: sum_u Z_tu B_u
                        zb += sZ[u * LQ + t] * sC[u * LS + s];  // dB_t: sum_u Z_ut C_u
                    }
                    float qhf = 0.f, qhb = 0.f, qgf = 0.f, qgb = 0.f;
                    for (int p = 0; p < P; ++p) {
                        const float yv = sY[t * LP + p], xv = sX[t * LP + p];
                        qhf += sHf[p * LL + tcol] * yv;
                        qhb += sHb[p * LL + tcol] * yv;
                        qgf += sGf[p * LL + tcol] * xv;
                        qgb += sGb[p * LL + tcol] * xv;
                    }
                    const float e_f = __expf(tk.cs[t]), e_b = __expf(tk.cs[Q - 1] - tk.ce[t]);
                    const int kk = sl * IPS + k2;
                    accC[kk] += zc + e_f * qhf + e_b * qhb;
                    accB[kk] += zb + tk.ef[t] * qgf + tk.eb[t] * qgb;
                    const float cv = sC[t * LS + s];
                    rf[k2] += cv * e_f * qhf;
                    rb[k2] += cv * e_b * qhb;
                }
            }
        }
        // rf, rb: sum over the SL columns (the SL lanes of a thread's row share t)
#pragma unroll
        for (int k2 = 0; k2 < IPS; ++k2) {
            const float vf = seg_sum(rf[k2], SL), vb = seg_sum(rb[k2], SL);
            const int t = trow + (NTB / SL) * k2;
            if (tcol == 0 && t < Q) {
                rfo[row + t] = vf;
                rbo[row + t] = vb;
            }
        }
    }
    const float inv_cnt = R > 0 ? 1.f / (float)(pt * ph * pw) : 0.f;
    for (int sl = 0; sl < nsl; ++sl) {
        const int s = sl * SL + tcol;
#pragma unroll
        for (int k2 = 0; k2 < IPS; ++k2) {
            const int t = trow + (NTB / SL) * k2;
            const uint32_t i = c * Q + t;
            if (t < Q && s < S && i < N) {
                const uint32_t n = rms_index32(i, order, T, H, W);
                const size_t o = ((b * N + n) * G + g) * S + s;
                float vb = accB[sl * IPS + k2];
                if (R > 0) vb += drBg[((b * R + review_of(n, rinv, H, W, pt, ph, pw)) * G + g) * S + s] * inv_cnt;
                elem<E>::store(dB + o, vb);
                elem<E>::store(dC + o, accC[sl * IPS + k2]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// ddt of one chunk and head, and its parts of dA and dD:
//   ddt_k = expl_k + A (span_f(k) + span_b(k)) (+ the review token's share),
//   span_f(k) = Sf(k) + sum_{t >= k} rf_t + sum_{u < k} cf_u + exp(tot) <Hf, Gf>,
//   span_b(k) = Sb(k) + sum_{t <= k} rb_t + sum_{u > k} cb_u + exp(tot) <Hb, Gb>,
// Sf(k) = sum_{j < k} (colsum of W below j - rowsum of W left of j),
// Sb(k) = sum_{j <= k} (rowsum of W right of j - colsum of W above j).
// grid (nch, nheads, batch), 256 threads; Q <= 64.
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(NTB) void k_bwd_ddt(const E *__restrict__ x, const E *__restrict__ dy,
                                                 const float *__restrict__ CB, const float *__restrict__ dtT,
                                                 const float *__restrict__ csT, const float *__restrict__ A,
                                                 const float *__restrict__ Hf, const float *__restrict__ Hb,
                                                 const float *__restrict__ Gf, const float *__restrict__ Gb,
                                                 const float *__restrict__ expl, const float *__restrict__ cfi,
                                                 const float *__restrict__ cbi, const float *__restrict__ rfi,
                                                 const float *__restrict__ rbi, const float *__restrict__ drdt,
                                                 const int *__restrict__ rinv, float *__restrict__ ddt,
                                                 float *__restrict__ pA, float *__restrict__ pD, int nheads, int P,
                                                 int S, int G, uint32_t N, uint32_t Lpad, int Q, int order, uint32_t T,
                                                 uint32_t H, uint32_t W, int pt, int ph, int pw, uint32_t R)
{
    extern __shared__ float sm[];
    const int LP = P + 1, LQ = Q + 1;
    float *sX = sm;                 // [Q][P+1]
    float *sY = sX + Q * LP;        // [Q][P+1]
    float *sW = sY + Q * LP;        // [Q][Q+1]  W_tu = M_tu (dy_t . x_u), t != u
    float *tkm = sW + Q * LQ;
    const TokLds tk{tkm, tkm + Q, tkm + 2 * Q, tkm + 3 * Q, tkm + 4 * Q};
    float *dj_f = tkm + 5 * Q, *dj_b = dj_f + Q;  // per-token increments of Sf and Sb
    float *red = dj_b + Q, *red2 = red + NTB;     // [NTB] each
    const uint32_t c = blockIdx.x, nch = gridDim.x;
    const int h = blockIdx.y, g = h / (nheads / G);
    const size_t b = blockIdx.z;
    const size_t row = (b * nheads + h) * Lpad + (size_t)c * Q;
    const float a = A[h];
    load_tokens(tk, dtT, csT, row, Q, a);
    load_rows(sX, LP, x, P, nheads, h, c, Q, N, b, order, T, H, W);
    load_rows(sY, LP, dy, P, nheads, h, c, Q, N, b, order, T, H, W);
    __syncthreads();
    const float *cb = CB + ((b * G + g) * nch + c) * (size_t)Q * Q;
    for (int k = threadIdx.x; k < Q * Q; k += NTB) {
        const int t = k / Q, u = k - t * Q;
        float w = 0.f;
        if (t != u) {
            float s_ = 0.f;
            for (int p = 0; p < P; ++p) s_ += sY[t * LP + p] * sX[u * LP + p];
            w = cb[k] * ldt(tk, t, u) * s_;
        }
        sW[t * LQ + u] = w;
    }
    // exp(tot) (<Hf, Gf> + <Hb, Gb>) and 2 x . dy over the chunk's tokens
    const size_t PS = (size_t)P * S, so = ((b * nheads + h) * nch + c) * PS;
    float cross = 0.f, xdy = 0.f;
    for (size_t e = threadIdx.x; e < PS; e += NTB) cross += Hf[so + e] * Gf[so + e] + Hb[so + e] * Gb[so + e];
    for (int e = threadIdx.x; e < Q * P; e += NTB) {  // positions past the end hold zeros
        const int u = e / P, p = e - u * P;
        xdy += sX[u * LP + p] * sY[u * LP + p];
    }
    red[threadIdx.x] = cross;
    red2[threadIdx.x] = xdy;
    __syncthreads();
    for (int j = threadIdx.x; j < Q; j += NTB) {
        float colb = 0.f, rowl = 0.f, rowr = 0.f, cola = 0.f;
        for (int t = j + 1; t < Q; ++t) colb += sW[t * LQ + j];
        for (int u = 0; u < j; ++u) rowl += sW[j * LQ + u];
        for (int u = j + 1; u < Q; ++u) rowr += sW[j * LQ + u];
        for (int t = 0; t < j; ++t) cola += sW[t * LQ + j];
        dj_f[j] = colb - rowl;
        dj_b[j] = rowr - cola;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float cr = 0.f, dD = 0.f;
        for (int k = 0; k < NTB; ++k) {
            cr += red[k];
            dD += red2[k];
        }
        cr *= __expf(tk.cs[Q - 1]);
        // sums over the chunk's tokens, taken in order
        float tot_rf = 0.f, tot_cb = 0.f;
        for (int k = 0; k < Q; ++k) {
            tot_rf += rfi[row + k];
            tot_cb += cbi[row + k];
        }
        float Sf = 0.f, Sb = 0.f, rf_ge = tot_rf, cf_lt = 0.f, rb_le = 0.f, cb_gt = tot_cb, dA = 0.f;
        const float inv_cnt = R > 0 ? 1.f / (float)(pt * ph * pw) : 0.f;
        for (int k = 0; k < Q; ++k) {
            Sb += dj_b[k];
            rb_le += rbi[row + k];
            cb_gt -= cbi[row + k];
            const float span = Sf + rf_ge + cf_lt + Sb + rb_le + cb_gt + cr;
            const uint32_t i = c * Q + k;
            if (i < N) {
                const uint32_t n = rms_index32(i, order, T, H, W);
                float v = expl[row + k] + a * span;
                if (R > 0) v += drdt[(b * R + review_of(n, rinv, H, W, pt, ph, pw)) * nheads + h] * inv_cnt;
                ddt[(b * N + n) * nheads + h] = v;
                dA += tk.dt[k] * span;
            }
            Sf += dj_f[k];
            rf_ge -= rfi[row + k];
            cf_lt += cfi[row + k];
        }
        pA[(b * nheads + h) * nch + c] = dA;
        pD[(b * nheads + h) * nch + c] = 2.f * dD;
    }
}

// dA[h], dD[h]: the chunks' and review tokens' parts summed over the batch. grid (ceil(nheads / 256)).
__global__ __launch_bounds__(256) void k_bwd_reduce(const float *__restrict__ pA, const float *__restrict__ pD,
                                                    const float *__restrict__ pAr, float *__restrict__ dA,
                                                    float *__restrict__ dD, int nheads, int nch, int batch)
{
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= nheads) return;
    float sa = 0.f, sd = 0.f;
    for (int b = 0; b < batch; ++b) {
        const size_t o = ((size_t)b * nheads + h) * nch;
        for (int c = 0; c < nch; ++c) {
            sa += pA[o + c];
            sd += pD[o + c];
        }
        if (pAr) sa += pAr[(size_t)b * nheads + h];
    }
    dA[h] = sa;
    dD[h] = sd;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// LDS floats of the dB/dC kernel (the largest of the per-chunk kernels) for chunk Q.
size_t dbdc_lds(int Q, int P, int S)
{
    return (size_t)2 * Q * (S + 1) + 2 * Q * (P + 1) + (size_t)Q * (Q + 1) + 4 * P * (SL + 1) + 5 * Q;
}

int bwd_chunk(const SsdProblem &p)
{
    return dbdc_lds(64, p.headdim, p.d_state) * 4 <= 150 * 1024 ? 64 : 32;
}

struct BwdLayout {
    int Q, nch, nchR;
    size_t dtT, csT, Sf, Sb, Uf, Ub, CB, expl, cf, cb, rf, rb, pA, pD;
    size_t rx, rB, rdt, rdtT, rcsT, rSf, rSb, h0f, h0b, Gf0, Gb0, drx, drB, drBg, drdt, pAr, rinv, total;
};

BwdLayout bwd_layout(const SsdProblem &p)
{
    BwdLayout l{};
    l.Q = bwd_chunk(p);
    l.nch = (int)((p.N + l.Q - 1) / l.Q);
    l.nchR = (int)((p.R + l.Q - 1) / l.Q);
    const size_t B = p.batch, Hs = p.nheads, PS = (size_t)p.headdim * p.d_state, G = p.ngroups;
    const size_t Lpad = (size_t)l.nch * l.Q;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    l.dtT = take(B * Hs * Lpad * 4);
    l.csT = take(B * Hs * Lpad * 4);
    l.Sf = take(B * Hs * l.nch * PS * 4);
    l.Sb = take(B * Hs * l.nch * PS * 4);
    l.Uf = take(B * Hs * l.nch * PS * 4);
    l.Ub = take(B * Hs * l.nch * PS * 4);
    l.CB = take(B * G * l.nch * (size_t)l.Q * l.Q * 4);
    l.expl = take(B * Hs * Lpad * 4);
    l.cf = take(B * Hs * Lpad * 4);
    l.cb = take(B * Hs * Lpad * 4);
    l.rf = take(B * Hs * Lpad * 4);
    l.rb = take(B * Hs * Lpad * 4);
    l.pA = take(B * Hs * l.nch * 4);
    l.pD = take(B * Hs * l.nch * 4);
    if (p.R > 0) {
        const size_t R = p.R, Rpad = (size_t)l.nchR * l.Q;
        l.rx = take(B * R * Hs * p.headdim * 4);
        l.rB = take(B * R * G * p.d_state * 4);
        l.rdt = take(B * R * Hs * 4);
        l.rdtT = take(B * Hs * Rpad * 4);
        l.rcsT = take(B * Hs * Rpad * 4);
        l.rSf = take(B * Hs * l.nchR * PS * 4);
        l.rSb = take(B * Hs * l.nchR * PS * 4);
        l.h0f = take(B * Hs * PS * 4);
        l.h0b = take(B * Hs * PS * 4);
        l.Gf0 = take(B * Hs * PS * 4);
        l.Gb0 = take(B * Hs * PS * 4);
        l.drx = take(B * R * Hs * p.headdim * 4);
        l.drB = take(B * R * Hs * p.d_state * 4);
        l.drBg = take(B * R * G * p.d_state * 4);
        l.drdt = take(B * R * Hs * 4);
        l.pAr = take(B * Hs * 4);
        l.rinv = take(R * 4);
    }
    l.total = off;
    return l;
}

size_t review_lds(const SsdProblem &p)
{
    return ((size_t)2 * p.headdim * p.d_state + p.headdim + p.d_state + 4 * (size_t)p.R + 2 * NTB) * 4;
}

template <typename E>
hipError_t run_backward(const SsdProblem &p, const SsdGradArgs &a, void *ws, hipStream_t st)
{
    const BwdLayout l = bwd_layout(p);
    char *w = (char *)ws;
    auto F = [&](size_t off) { return (float *)(w + off); };
    float *dtT = F(l.dtT), *csT = F(l.csT), *Sf = F(l.Sf), *Sb = F(l.Sb), *Uf = F(l.Uf), *Ub = F(l.Ub);
    float *CB = F(l.CB), *expl = F(l.expl), *cf = F(l.cf), *cb = F(l.cb), *rf = F(l.rf), *rb = F(l.rb);
    float *pA = F(l.pA), *pD = F(l.pD);
    const int Hs = p.nheads, P = p.headdim, S = p.d_state, G = p.ngroups, Q = l.Q;
    const uint32_t N = (uint32_t)p.N, Lpad = (uint32_t)(l.nch * Q);
    const uint32_t T = (uint32_t)p.T, H = (uint32_t)p.H, W = (uint32_t)p.W;
    const int B = (int)p.batch;
    const E *x = (const E *)a.x, *Bm = (const E *)a.b, *Cm = (const E *)a.c, *dy = (const E *)a.dy;
    const size_t states_lds = ((size_t)Q * P + (size_t)Q * S + 2 * Q) * 4;
    const uint32_t R = (uint32_t)p.R;
    timing::Scope ts_(K_SSD_BWD, st);

    float *h0f = nullptr, *h0b = nullptr, *Gf0 = nullptr, *Gb0 = nullptr, *drx = nullptr, *drBg = nullptr,
          *drdt = nullptr, *pAr = nullptr;
    int *rinv = nullptr;
    if (R > 0) {
        float *rx = F(l.rx), *rB = F(l.rB), *rdt = F(l.rdt), *rdtT = F(l.rdtT), *rcsT = F(l.rcsT);
        float *rSf = F(l.rSf), *rSb = F(l.rSb);
        h0f = F(l.h0f);
        h0b = F(l.h0b);
        const uint32_t Rpad = (uint32_t)(l.nchR * Q);
        const int64_t Cx = (int64_t)Hs * P, Cbw = (int64_t)G * S;
        k_pool<E, float><<<dim3((Cx + 255) / 256, R, B), 256, 0, st>>>(x, rx, Cx, T, H, W, p.pool_t, p.pool_h, p.pool_w,
                                                                       p.order);
        k_pool<E, float><<<dim3((Cbw + 255) / 256, R, B), 256, 0, st>>>(Bm, rB, Cbw, T, H, W, p.pool_t, p.pool_h,
                                                                        p.pool_w, p.order);
        k_pool<float, float><<<dim3((Hs + 255) / 256, R, B), 256, 0, st>>>(a.dt, rdt, Hs, T, H, W, p.pool_t, p.pool_h,
                                                                          p.pool_w, p.order);
        k_prep_dt<false><<<dim3(l.nchR, (Hs + 63) / 64, B), 256, 0, st>>>(rdt, a.a, rdtT, rcsT, Hs, R, Rpad, Q, 0, 1, 1,
                                                                         R);
        k_chunk_states<float, false, false><<<dim3(l.nchR, Hs, B), 256, states_lds, st>>>(
            rx, rB, rdtT, rcsT, a.a, rSf, rSb, Hs, P, S, G, R, Rpad, Q, 0, 1, 1, R);
        k_state_pass<<<dim3((P * S + 255) / 256, Hs, B), 256, 0, st>>>(rSf, rSb, rcsT, nullptr, nullptr, h0f, h0b,
                                                                      P * S, l.nchR, Q, Rpad);
        rinv = (int *)(w + l.rinv);
        k_review_index<<<(R + 255) / 256, 256, 0, st>>>(rinv, R, p.order, T / p.pool_t, H / p.pool_h, W / p.pool_w);
        Gf0 = F(l.Gf0);
        Gb0 = F(l.Gb0);
        drx = F(l.drx);
        drBg = F(l.drBg);
        drdt = F(l.drdt);
        pAr = F(l.pAr);
    }
    k_prep_dt<true><<<dim3(l.nch, (Hs + 63) / 64, B), 256, 0, st>>>(a.dt, a.a, dtT, csT, Hs, N, Lpad, Q, p.order, T,
                                                                    H, W);
    // states of the forward pass (entering each chunk), then the adjoint states
    k_chunk_states<E, true, false><<<dim3(l.nch, Hs, B), 256, states_lds, st>>>(x, Bm, dtT, csT, a.a, Sf, Sb, Hs, P, S,
                                                                               G, N, Lpad, Q, p.order, T, H, W);
    k_state_pass<<<dim3((P * S + 255) / 256, Hs, B), 256, 0, st>>>(Sf, Sb, csT, h0f, h0b, nullptr, nullptr, P * S,
                                                                  l.nch, Q, Lpad);
    k_chunk_states<E, true, true><<<dim3(l.nch, Hs, B), 256, states_lds, st>>>(dy, Cm, dtT, csT, a.a, Uf, Ub, Hs, P, S,
                                                                              G, N, Lpad, Q, p.order, T, H, W);
    // Ub runs left to right (Gb, from the chunks before), Uf right to left (Gf, from the chunks after); the
    // final values are the adjoints of the review tokens' states.
    k_state_pass<<<dim3((P * S + 255) / 256, Hs, B), 256, 0, st>>>(Ub, Uf, csT, nullptr, nullptr, Gb0, Gf0, P * S,
                                                                  l.nch, Q, Lpad);
    k_cb<E><<<dim3(l.nch, G, B), 256, 0, st>>>(Bm, Cm, CB, G, S, N, Q, p.order, T, H, W);
    if (R > 0) {
        k_review_grads<<<B * Hs, NTB, review_lds(p), st>>>(F(l.rx), F(l.rB), F(l.rdt), a.a, Gf0, Gb0, drx, F(l.drB),
                                                           drdt, pAr, Hs, P, S, G, (int)R);
        k_review_group<<<dim3(R, B), 256, 0, st>>>(F(l.drB), drBg, Hs, S, G);
    }
    const size_t lds_dx =
        ((size_t)Q * (Q + 1) + 2 * (size_t)Q * (P + 1) + (size_t)Q * (S + 1) + 2 * P * (SL + 1) + 8 * Q) * 4;
    k_bwd_dx<E><<<dim3(l.nch, Hs, B), NTB, lds_dx, st>>>(x, dy, Bm, CB, dtT, csT, a.a, a.d, Uf, Ub, drx, rinv,
                                                        (E *)a.dx, expl, cf, cb, Hs, P, S, G, N, Lpad, Q, p.order, T,
                                                        H, W, p.pool_t, p.pool_h, p.pool_w, R);
    k_bwd_dbdc<E><<<dim3(l.nch, G, B), NTB, dbdc_lds(Q, P, S) * 4, st>>>(
        x, dy, Bm, Cm, dtT, csT, a.a, Sf, Sb, Uf, Ub, drBg, rinv, (E *)a.db, (E *)a.dc, rf, rb, Hs, P, S, G, N, Lpad,
        Q, p.order, T, H, W, p.pool_t, p.pool_h, p.pool_w, R);
    const size_t lds_ddt = (2 * (size_t)Q * (P + 1) + (size_t)Q * (Q + 1) + 7 * Q + 2 * NTB) * 4;
    k_bwd_ddt<E><<<dim3(l.nch, Hs, B), NTB, lds_ddt, st>>>(x, dy, CB, dtT, csT, a.a, Sf, Sb, Uf, Ub, expl, cf, cb, rf,
                                                          rb, drdt, rinv, a.ddt, pA, pD, Hs, P, S, G, N, Lpad, Q,
                                                          p.order, T, H, W, p.pool_t, p.pool_h, p.pool_w, R);
    k_bwd_reduce<<<(Hs + 255) / 256, 256, 0, st>>>(pA, pD, pAr, a.da, a.dd, Hs, l.nch, B);
    return hipGetLastError();
}

template <typename E>
hipError_t set_lds_attrs()
{
    const int lds = 160 * 1024;
    hipError_t e;
    if ((e = hipFuncSetAttribute((const void *)k_chunk_states<E, true, false>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_chunk_states<E, true, true>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_bwd_dx<E>, hipFuncAttributeMaxDynamicSharedMemorySize, lds)) !=
        hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_bwd_dbdc<E>, hipFuncAttributeMaxDynamicSharedMemorySize, lds)) !=
        hipSuccess) return e;
    return hipFuncSetAttribute((const void *)k_bwd_ddt<E>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

} // namespace

bool ssd_backward_supports(const SsdProblem &p)
{
    return (p.headdim == 16 || p.headdim == 32 || p.headdim == 64) && p.d_state <= 128 && p.d_state % 8 == 0 &&
           (size_t)review_lds(p) <= 160 * 1024;
}

size_t ssd_backward_workspace(const SsdProblem &p) { return bwd_layout(p).total; }

hipError_t ssd_backward_prepare()
{
    hipError_t e;
    if ((e = set_lds_attrs<float>()) != hipSuccess) return e;
    if ((e = set_lds_attrs<bf16_t>()) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_chunk_states<float, false, false>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024)) != hipSuccess) return e;
    return hipFuncSetAttribute((const void *)k_review_grads, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

hipError_t ssd_backward(const SsdProblem &p, const SsdGradArgs &a, void *ws, hipStream_t st)
{
    if (p.dtype == 0) return run_backward<float>(p, a, ws, st);
    return run_backward<bf16_t>(p, a, ws, st);
}

} // namespace mate
