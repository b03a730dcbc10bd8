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
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "mfma_frag.hpp"
#include "ssd_chunks.hpp"
#include "ssd_common.hpp"
#include "timing.hpp"

namespace mate {

namespace {

using ssd::k_cb;
using ssd::k_chunk_states;
using ssd::k_pool;
using ssd::prep_dt;
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
// Gradients of the review tokens of one (batch, head), RT tokens per workgroup. Forward direction: the
// adjoint of the state the review tokens leave to the main sequence is Gf0; a review token r reaches it
// with decay df_r = exp(sum_{j > r} dt_j A). Backward direction (review tokens taken in reverse order):
// Gb0 and db_r = exp(sum_{j < r} dt_j A). dy is 0 on review tokens, so each token's pairs are with main
// tokens only, and the pairs spanning r are those whose review end lies before r in that direction:
// this kernel writes each token's pair sums (cfr, cbr) and the explicit part of its dt gradient;
// k_review_spans adds the spans. grid (ceil(R / RT) * batch * nheads), 256 threads; P <= 64, S <= 128.
// ---------------------------------------------------------------------------
constexpr int RT = 16;  // review tokens per workgroup

__global__ __launch_bounds__(NTB) void k_review_grads(const float *__restrict__ rx, const float *__restrict__ rB,
                                                      const float *__restrict__ rdt, const float *__restrict__ A,
                                                      const float *__restrict__ Gf0, const float *__restrict__ Gb0,
                                                      float *__restrict__ drx, float *__restrict__ drB,
                                                      float *__restrict__ drdt, float *__restrict__ cfr,
                                                      float *__restrict__ cbr, int nheads, int P, int S, int G, int R)
{
    extern __shared__ float sm[];
    const int PS = P * S;
    float *gf = sm, *gb = gf + PS;             // adjoint states [P][S]
    float *xs = gb + PS, *bs = xs + P;         // the token's x and B
    float *decf = bs + S, *decb = decf + RT;   // decays to the review end, per direction
    float *red = decb + RT;                    // [2][NTB] partial sums
    const int nrb = (R + RT - 1) / RT;
    const int bh = blockIdx.x / nrb, b = bh / nheads, h = bh % nheads, g = h / (nheads / G);
    const int r0 = (blockIdx.x % nrb) * RT, r1 = min(R, r0 + RT);
    const float a = A[h];
    for (int e = threadIdx.x; e < PS; e += NTB) {
        gf[e] = Gf0[(size_t)bh * PS + e];
        gb[e] = Gb0[(size_t)bh * PS + e];
    }
    if (threadIdx.x == 0) {
        float run = 1.f;
        for (int r = R - 1; r >= r0; --r) {
            if (r < r1) decf[r - r0] = run;
            run *= __expf(rdt[((size_t)b * R + r) * nheads + h] * a);
        }
        run = 1.f;
        for (int r = 0; r < r1; ++r) {
            if (r >= r0) decb[r - r0] = run;
            run *= __expf(rdt[((size_t)b * R + r) * nheads + h] * a);
        }
    }
    __syncthreads();
    // thread layout: for G x B (P outputs), 4 threads per p split S; for G^T x (S outputs), 2 threads per s split P
    const int tp = threadIdx.x >> 2, tq = threadIdx.x & 3;
    const int ts = threadIdx.x >> 1, tr = threadIdx.x & 1;
    for (int r = r0; r < r1; ++r) {
        const float d = rdt[((size_t)b * R + r) * nheads + h];
        const float df = decf[r - r0], db = decb[r - r0];
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
            const float vf = df * pf, vb = db * pb;
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
        if (ts < S && tr == 0) drB[(((size_t)b * R + r) * nheads + h) * S + ts] = d * (df * qf + db * qb);
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
            drdt[((size_t)b * R + r) * nheads + h] = ef + eb;  // explicit part; k_review_spans adds the decay part
            cfr[(size_t)bh * R + r] = d * ef;
            cbr[(size_t)bh * R + r] = d * eb;
        }
        __syncthreads();
    }
}

// The decay part of the review tokens' dt gradients and their share of dA: forward pairs spanning r have
// their review end u < r, backward pairs u > r. grid (ceil(batch * nheads / 256)).
__global__ __launch_bounds__(256) void k_review_spans(const float *__restrict__ rdt, const float *__restrict__ A,
                                                      const float *__restrict__ cfr, const float *__restrict__ cbr,
                                                      float *__restrict__ drdt, float *__restrict__ pAr, int nheads,
                                                      int R, int nbh)
{
    const int bh = blockIdx.x * 256 + threadIdx.x;
    if (bh >= nbh) return;
    const int b = bh / nheads, h = bh % nheads;
    const float a = A[h];
    float below = 0.f, dA = 0.f;
    for (int r = 0; r < R; ++r) {
        float *o = drdt + ((size_t)b * R + r) * nheads + h;
        *o += a * below;
        dA += rdt[((size_t)b * R + r) * nheads + h] * below;
        below += cfr[(size_t)bh * R + r];
    }
    float above = 0.f;
    for (int r = R - 1; r >= 0; --r) {
        float *o = drdt + ((size_t)b * R + r) * nheads + h;
        *o += a * above;
        dA += rdt[((size_t)b * R + r) * nheads + h] * above;
        above += cbr[(size_t)bh * R + r];
    }
    pAr[bh] = dA;
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

// ---------------------------------------------------------------------------
// MFMA kernels (bf16 tensors, headdim 64, d_state 64 or 128, chunks of 64): the
// same chunked evaluation with every product on v_mfma_f32_32x32x16_bf16 and
// fp32 accumulation. The tensors are bf16 already; the fp32 states enter the
// products rounded to bf16, and the intra-chunk matrices M and Z, whose large
// near-diagonal entries would otherwise dominate the error, as a pair of bf16
// terms (hi = bf16(m), lo = bf16(m - hi)), i.e. to about 16 bits.
// ---------------------------------------------------------------------------
using frag::acc_row;
using frag::bf16x8;
using frag::f32x16;
using frag::frag_rm;
using frag::frag_tr;
using frag::mfma_bf16;

constexpr int QM = 64;         // chunk
constexpr int PM = 64;         // head dim
constexpr int LXM = PM + 8;    // row stride of [64][64] bf16 tiles
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// L_tu without branches (the exponent is selected first, so the other direction's never overflows).
__device__ __forceinline__ float ldt_sel(const TokLds &tk, int t, int u)
{
    const float arg = u < t ? tk.cs[t] - tk.cs[u] : tk.ce[u] - tk.ce[t];
    const float v = tk.dt[u] * __expf(arg);
    return u == t ? 2.f * tk.dt[t] : v;
}

// Workgroup barrier for data exchanged through LDS: waits for this wave's LDS operations only, so global
// loads issued ahead (prefetches into registers) stay in flight across it. Everything the MFMA kernels
// share between waves is written to LDS explicitly.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr uint32_t kNoToken = 0xffffffffu;

// Canonical token index of each scan position of chunk c (kNoToken past the end) and, with review tokens
// (R > 0), the review token of its pool block. The caller synchronises before the indices are read.
__device__ __forceinline__ void chunk_tokens(uint32_t *s_n, uint32_t *s_rv, uint32_t c, uint32_t N, int order,
                                             uint32_t T, uint32_t H, uint32_t W, const int *rinv, int pt, int ph,
                                             int pw, uint32_t R)
{
    for (int u = threadIdx.x; u < QM; u += NTB) {
        const uint32_t i = c * QM + u;
        uint32_t n = kNoToken, r = 0;
        if (i < N) {
            n = rms_index32(i, order, T, H, W);
            if (R > 0) r = review_of(n, rinv, H, W, pt, ph, pw);
        }
        s_n[u] = n;
        if (s_rv) s_rv[u] = r;
    }
}

// 16-byte pieces of the chunk's token rows (COLS bf16 channels of head/group hd of nh, the tokens given
// by s_n; zeros past the end) into registers, NTH threads sharing the QM x COLS tile ...
template <int COLS, int NTH>
__device__ __forceinline__ void fetch_rows(u32x4v (&r)[QM * COLS / 8 / NTH], const __bf16 *src, int nh, int hd,
                                           const uint32_t *s_n, size_t b, uint32_t N)
{
    constexpr int PPR = COLS / 8;  // pieces per row
    static_assert(QM * PPR % NTH == 0, "row pieces");
#pragma unroll
    for (int j = 0; j < QM * PPR / NTH; ++j) {
        const int k = threadIdx.x + NTH * j, u = k / PPR, pc = k % PPR;
        const uint32_t n = s_n[u];
        // an unconditional load (token 0's row past the end, zeroed when stored): no branch around it
        r[j] = *(const u32x4v *)(src + ((b * N + (n == kNoToken ? 0u : n)) * nh + hd) * COLS + 8 * pc);
    }
}

// ... and from registers into an LDS tile of row stride ld (rows past the end as zeros).
template <int COLS, int NTH>
__device__ __forceinline__ void store_rows(__bf16 *dst, int ld, const u32x4v (&r)[QM * COLS / 8 / NTH],
                                           const uint32_t *s_n)
{
    constexpr int PPR = COLS / 8;
#pragma unroll
    for (int j = 0; j < QM * PPR / NTH; ++j) {
        const int k = threadIdx.x + NTH * j, u = k / PPR, pc = k % PPR;
        *(u32x4v *)(dst + u * ld + 8 * pc) = s_n[u] == kNoToken ? u32x4v{0, 0, 0, 0} : r[j];
    }
}

template <int COLS, int NTH>
__device__ __forceinline__ void load_rows_tok(__bf16 *dst, int ld, const __bf16 *src, int nh, int hd,
                                              const uint32_t *s_n, size_t b, uint32_t N)
{
    u32x4v r[QM * COLS / 8 / NTH];
    fetch_rows<COLS, NTH>(r, src, nh, hd, s_n, b, N);
    store_rows<COLS, NTH>(dst, ld, r, s_n);
}

// Block -> (chunk c, head h) with all heads of a chunk on one XCD, so that the chunk's B and C rows are
// fetched into that XCD's L2 once: blocks are handed to the 8 XCDs in turn (block id mod 8), and block
// id = 8 (nheads grp + h) + k takes chunk 8 grp + k. Returns false for the padding past the last chunk.
__device__ __forceinline__ bool chunk_head_of(uint32_t nch, int nheads, uint32_t &c, int &h)
{
    const uint32_t id = blockIdx.x, q = id >> 3;
    h = (int)(q % (uint32_t)nheads);
    c = 8 * (q / (uint32_t)nheads) + (id & 7);
    return c < nch;
}

// Sums over the 32 lanes of each half-wave of the 16 values v[e] (one per accumulator row of a 32 x 32
// tile). Halving exchanges: after them lane j of the half holds the total of value (j >> 1) & 15.
__device__ __forceinline__ float half_sum16(const float (&v)[16])
{
    const int l = threadIdx.x & 63;
    float a8[8], a4[4], a2[2];
    const bool b4 = l & 16, b3 = l & 8, b2 = l & 4, b1 = l & 2;
#pragma unroll
    for (int k = 0; k < 8; ++k) a8[k] = (b4 ? v[k + 8] : v[k]) + __shfl_xor(b4 ? v[k] : v[k + 8], 16, 64);
#pragma unroll
    for (int k = 0; k < 4; ++k) a4[k] = (b3 ? a8[k + 4] : a8[k]) + __shfl_xor(b3 ? a8[k] : a8[k + 4], 8, 64);
#pragma unroll
    for (int k = 0; k < 2; ++k) a2[k] = (b2 ? a4[k + 2] : a4[k]) + __shfl_xor(b2 ? a4[k] : a4[k + 2], 4, 64);
    const float a1 = (b1 ? a2[1] : a2[0]) + __shfl_xor(b1 ? a2[0] : a2[1], 2, 64);
    return a1 + __shfl_xor(a1, 1, 64);
}

// Sum of v over the NTH threads of the block (every thread gets it); red holds NTH / 64 floats.
template <int NTH>
__device__ __forceinline__ float block_sum(float v, float *red)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    lds_barrier();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    lds_barrier();
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < NTH / 64; ++k) t += red[k];
    return t;
}

// ---------------------------------------------------------------------------
// Chunk contributions of the states (ADJ false: x, B) or the adjoint states (ADJ true: dy, C) on MFMA:
// Sf = X^T diag(wf) B, Sb = X^T diag(wb) B (P x S, stored bf16), the weights as in k_chunk_states, applied
// to the X^T operand in registers. Waves 0-1 make Sf, waves 2-3 Sb, S/32 tiles each.
// grid (8 nheads ceil(nch / 8), batch), 256 threads (chunk and head as in chunk_head_of).
// ---------------------------------------------------------------------------
template <int S, bool ADJ>
__global__ __launch_bounds__(NTB) void k_bwd_states_mfma(const __bf16 *__restrict__ x, const __bf16 *__restrict__ Bm,
                                                         const float *__restrict__ dtT, const float *__restrict__ csT,
                                                         const float *__restrict__ A, __bf16 *__restrict__ Sf,
                                                         __bf16 *__restrict__ Sb, int nheads, int G, uint32_t N,
                                                         uint32_t Lpad, uint32_t nch, int order, uint32_t T,
                                                         uint32_t H, uint32_t W)
{
    constexpr int LS = S + 8, NT = S / 32, TPW = S / 32;
    constexpr int LG = 72;  // row pitch of a wave's output staging (64 columns + 8)
    static_assert(TPW % 2 == 0, "tiles are staged two at a time");
    __shared__ __attribute__((aligned(16))) __bf16 sX[QM * LXM];
    // B rows; after the products, each wave's output staging
    __shared__ __attribute__((aligned(16))) __bf16 sB[QM * LS > 4 * 32 * LG ? QM * LS : 4 * 32 * LG];
    __shared__ float s_w[2][QM];
    __shared__ uint32_t s_n[QM];
    uint32_t c;
    int h;
    if (!chunk_head_of(nch, nheads, c, h)) return;
    const int g = h / (nheads / G);
    const size_t b = blockIdx.y;
    const size_t row = (b * nheads + h) * Lpad + (size_t)c * QM;
    const float a = A[h];
    chunk_tokens(s_n, nullptr, c, N, order, T, H, W, nullptr, 1, 1, 1, 0);
    lds_barrier();
    load_rows_tok<PM, NTB>(sX, LXM, x, nheads, h, s_n, b, N);
    load_rows_tok<S, NTB>(sB, LS, Bm, G, g, s_n, b, N);
    {
        const float tot = csT[row + QM - 1];
        for (int u = threadIdx.x; u < QM; u += NTB) {
            const float d = dtT[row + u], cs = csT[row + u];
            s_w[0][u] = ADJ ? __expf(cs) : d * __expf(tot - cs);
            s_w[1][u] = ADJ ? __expf(tot - (cs - d * a)) : d * __expf(cs - d * a);
        }
    }
    lds_barrier();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int which = wave >> 1;  // 0: Sf, 1: Sb
    __bf16 *out = (which ? Sb : Sf) + ((b * nheads + h) * nch + c) * (size_t)(PM * S);
    f32x16 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = f32x16{};
#pragma unroll
    for (int k0 = 0; k0 < QM; k0 += 16) {
        float w8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w8[j] = s_w[which][k0 + 8 * (lane >> 5) + j];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tile = (wave & 1) * TPW + i, mt = tile / NT, nt = tile % NT;
            bf16x8 af = frag_tr(sX, LXM, k0, 32 * mt);  // X^T[p][u]
#pragma unroll
            for (int j = 0; j < 8; ++j) af[j] = (__bf16)((float)af[j] * w8[j]);
            acc[i] = mfma_bf16(af, frag_tr(sB, LS, k0, 32 * nt), acc[i]);
        }
    }
    // The wave's tiles are rows 32 mt .. 32 mt + 31 of the output (mt = wave % 2), all S columns: they
    // leave through LDS, two tiles (64 columns) at a time, as 16-byte row pieces.
    typedef uint32_t piece __attribute__((ext_vector_type(4)));
    lds_barrier();  // every wave is done with sX and sB
    __bf16 *stg = sB + wave * (32 * LG);
    const int mt = wave & 1;
#pragma unroll
    for (int r = 0; r < TPW / 2; ++r) {
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int e = 0; e < 16; ++e) stg[acc_row(e, lane) * LG + 32 * i2 + (lane & 31)] = (__bf16)acc[2 * r + i2][e];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int idx = lane + 64 * k, rr = idx >> 3, pc = idx & 7;
            *(piece *)(out + (size_t)(32 * mt + rr) * S + 64 * r + 8 * pc) = *(const piece *)(stg + rr * LG + 8 * pc);
        }
    }
}

// ---------------------------------------------------------------------------
// Turns bf16 chunk contributions into the bf16 states entering each chunk, in place, with the running
// state in fp32: the even blockIdx.y of a head runs left to right over Sf (Sf[c] becomes the state after
// chunk c - 1), the odd one right to left over Sb (the state after chunk c + 1). h0f / h0b (optional) are
// the initial states, finF / finB (optional) receive the final ones, fp32 [batch][nheads][P*S]. Each
// thread carries 8 consecutive elements through batches of U chunks; a batch's loads are issued before
// the previous batch's updates and stores, so waiting for them never waits for those stores (the memory
// counter retires in issue order). grid (ceil(P*S / 2048), 2 nheads, batch), 256 threads; P*S a multiple
// of 8.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_state_pass_bf16(__bf16 *__restrict__ Sf, __bf16 *__restrict__ Sb,
                                                         const float *__restrict__ csT, const float *__restrict__ h0f,
                                                         const float *__restrict__ h0b, float *__restrict__ finF,
                                                         float *__restrict__ finB, int PS, int nch, uint32_t Lpad)
{
    constexpr int U = 8;
    const int e = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (e >= PS) return;
    const int h = blockIdx.y >> 1, dir = blockIdx.y & 1;
    const size_t bh = (size_t)blockIdx.z * (gridDim.y >> 1) + h;
    const float *tot = csT + bh * Lpad + (QM - 1);
    __bf16 *base = (dir ? Sb : Sf) + bh * nch * (size_t)PS + e;
    const float *h0 = dir ? h0b : h0f;
    float *fin = dir ? finB : finF;
    float run[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) run[j] = h0 ? h0[bh * PS + e + j] : 0.f;
    // chunk of batch position k of the batch starting at c0 (clamped: loads past the end repeat the last
    // chunk and are not used)
    auto chunk = [&](int c0, int k) {
        const int i = min(c0 + k, nch - 1);
        return dir ? nch - 1 - i : i;
    };
    // two register sets, used alternately (static indices: the loop body covers one batch in each)
    bf16x8 va[U], vb[U];
    float da[U], db[U];
    auto load = [&](int c0, bf16x8 (&v)[U], float (&d)[U]) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int c = chunk(c0, k);
            v[k] = *(const bf16x8 *)(base + (size_t)c * PS);
            d[k] = __expf(tot[(size_t)c * QM]);
        }
    };
    auto update = [&](int c0, const bf16x8 (&v)[U], const float (&d)[U]) {
        const int n = min(U, nch - c0);
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (k < n) {
                bf16x8 o;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    o[j] = (__bf16)run[j];
                    run[j] = d[k] * run[j] + (float)v[k][j];
                }
                *(bf16x8 *)(base + (size_t)chunk(c0, k) * PS) = o;
            }
        }
    };
    load(0, va, da);
    for (int c0 = 0; c0 < nch; c0 += 2 * U) {
        if (c0 + U < nch) load(c0 + U, vb, db);
        update(c0, va, da);
        if (c0 + U >= nch) break;
        if (c0 + 2 * U < nch) load(c0 + 2 * U, va, da);
        update(c0 + U, vb, db);
    }
    if (fin)
#pragma unroll
        for (int j = 0; j < 8; ++j) fin[bh * PS + e + j] = run[j];
}

// ---------------------------------------------------------------------------
// dB and dC of one chunk and group on MFMA, the group's heads in turn (sums in accumulators), with each
// head's rf_t = exp(cs_t) C_t . (Hf^T dy_t), rb_t = exp(tot - ce_t) C_t . (Hb^T dy_t) and its
// cross term exp(tot) (<Hf, Gf> + <Hb, Gb>) (fp32 sums of the stored bf16 states). Per head: DX = dy x^T and
// Z = DX o L (to LDS), then for the wave's output tile (rows: tokens, columns: state)
//   dC[t][s] += (Z B)[t][s] + exp(cs_t) (dy Hf)[t][s] + exp(tot - ce_t) (dy Hb)[t][s],
//   dB[u][s] += (Z^T C)[u][s] + ef_u (x Gf)[u][s] + eb_u (x Gb)[u][s].
// The next head's operands are fetched into registers while this one computes.
// grid (nch, G, batch), S / 16 waves (one 32 x 32 tile of dB and of dC each).
// ---------------------------------------------------------------------------
template <int S>
__global__ __launch_bounds__(4 * S) void k_bwd_dbdc_mfma(const __bf16 *__restrict__ x, const __bf16 *__restrict__ dy,
                                                         const __bf16 *__restrict__ Bm, const __bf16 *__restrict__ Cm,
                                                         const float *__restrict__ dtT, const float *__restrict__ csT,
                                                         const float *__restrict__ A, const __bf16 *__restrict__ Hf,
                                                         const __bf16 *__restrict__ Hb, const __bf16 *__restrict__ Gf,
                                                         const __bf16 *__restrict__ Gb, const float *__restrict__ drBg,
                                                         const int *__restrict__ rinv, __bf16 *__restrict__ dB,
                                                         __bf16 *__restrict__ dC, float *__restrict__ rfo,
                                                         float *__restrict__ rbo, float *__restrict__ crs, int nheads,
                                                         int G, uint32_t N, uint32_t Lpad, int order, uint32_t T,
                                                         uint32_t H, uint32_t W, int pt, int ph, int pw, uint32_t R)
{
    constexpr int LS = S + 8, NT = S / 32, NTH = 4 * S;  // 2 NT tiles of 32 x 32, a wave each
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    __bf16 *sB = (__bf16 *)smem_raw;       // [Q][LS]
    __bf16 *sC = sB + QM * LS;             // [Q][LS]
    __bf16 *sX = sC + QM * LS;             // [Q][LXM]
    __bf16 *sY = sX + QM * LXM;            // [Q][LXM]
    __bf16 *sZ = sY + QM * LXM;            // 2 x [Q][LXM]  Z_tu as bf16 hi + lo
    __bf16 *sH = sZ + 2 * QM * LXM;        // 4 x [P][LS]: Hf, Hb, Gf, Gb
    float *tkm = (float *)(sH + 4 * PM * LS);
    const TokLds tk{tkm, tkm + QM, tkm + 2 * QM, tkm + 3 * QM, tkm + 4 * QM};
    float *s_rp = tkm + 5 * QM;            // [2][NT][Q] partial row sums of rf, rb
    float *s_red = s_rp + 2 * NT * QM;     // [NTH / 64]
    __shared__ uint32_t s_n[QM], s_rv[QM];
    const uint32_t c = blockIdx.x, nch = gridDim.x;
    const int g = blockIdx.y, hpg = nheads / G;
    const size_t b = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int mt = wave / NT, nt = wave % NT;  // this wave's tile: tokens 32 mt + .., state columns 32 nt + ..
    chunk_tokens(s_n, s_rv, c, N, order, T, H, W, rinv, pt, ph, pw, R);
    lds_barrier();
    load_rows_tok<S, NTH>(sB, LS, Bm, G, g, s_n, b, N);
    load_rows_tok<S, NTH>(sC, LS, Cm, G, g, s_n, b, N);
    f32x16 accB = f32x16{}, accC = f32x16{};
    const size_t PS = (size_t)PM * S;
    // A head's operands are fetched into registers (the next head's while this one computes), then staged
    // in LDS: the four states, the x and dy rows, and the tokens' dt and cumulative sums.
    constexpr int NPS = PM * S / 8 / NTH, NPX = QM * PM / 8 / NTH;  // 16-byte pieces per thread
    static_assert(NPS * NTH * 8 == PM * S, "state pieces");
    bf16x8 rh[4][NPS];
    u32x4v rx[NPX], ry[NPX];
    float rdt = 0.f, rcs = 0.f, rtot = 0.f;
    auto fetch = [&](int h) {
        const size_t so = ((b * nheads + h) * nch + c) * PS;
        const __bf16 *src[4] = {Hf + so, Hb + so, Gf + so, Gb + so};
#pragma unroll
        for (int j = 0; j < NPS; ++j) {
            const int k = threadIdx.x + NTH * j, pp = k / (S / 8), s8 = 8 * (k % (S / 8));
#pragma unroll
            for (int q = 0; q < 4; ++q) rh[q][j] = *(const bf16x8 *)(src[q] + (size_t)pp * S + s8);
        }
        fetch_rows<PM, NTH>(rx, x, nheads, h, s_n, b, N);
        fetch_rows<PM, NTH>(ry, dy, nheads, h, s_n, b, N);
        const size_t row = (b * nheads + h) * Lpad + (size_t)c * QM;
        const int u = threadIdx.x & (QM - 1);  // the tokens' values (threads past QM load duplicates)
        rdt = dtT[row + u];
        rcs = csT[row + u];
        rtot = csT[row + QM - 1];
    };
    // stores the fetched head into LDS; returns this thread's part of <Hf, Gf> + <Hb, Gb>
    auto stage = [&](int h) {
        float cross = 0.f;
#pragma unroll
        for (int j = 0; j < NPS; ++j) {
            const int k = threadIdx.x + NTH * j, pp = k / (S / 8), s8 = 8 * (k % (S / 8));
#pragma unroll
            for (int e = 0; e < 8; ++e)
                cross += (float)rh[0][j][e] * (float)rh[2][j][e] + (float)rh[1][j][e] * (float)rh[3][j][e];
#pragma unroll
            for (int q = 0; q < 4; ++q) *(bf16x8 *)(sH + q * PM * LS + pp * LS + s8) = rh[q][j];
        }
        store_rows<PM, NTH>(sX, LXM, rx, s_n);
        store_rows<PM, NTH>(sY, LXM, ry, s_n);
        if (threadIdx.x < QM) {
            const int u = threadIdx.x;
            const float ce = rcs - rdt * A[h];
            tk.dt[u] = rdt;
            tk.cs[u] = rcs;
            tk.ce[u] = ce;
            tk.ef[u] = rdt * __expf(rtot - rcs);
            tk.eb[u] = rdt * __expf(ce);
        }
        return cross;
    };
    fetch(g * hpg);
    float cr = stage(g * hpg);
    for (int hk = 0; hk < hpg; ++hk) {
        const int h = g * hpg + hk;
        const size_t row = (b * nheads + h) * Lpad + (size_t)c * QM;
        lds_barrier();  // this head's operands are staged
        if (hk + 1 < hpg) fetch(h + 1);
        if (wave < 4) {  // DX tile (t, u) of this wave, then Z = DX o L into LDS
            const int dm = wave >> 1, dn = wave & 1;
            f32x16 d = f32x16{};
#pragma unroll
            for (int k0 = 0; k0 < PM; k0 += 16)
                d = mfma_bf16(frag_rm(sY, LXM, 32 * dm, k0), frag_rm(sX, LXM, 32 * dn, k0), d);
            const int u = 32 * dn + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = 32 * dm + acc_row(e, lane);
                const float z = d[e] * ldt_sel(tk, t, u);
                const __bf16 hi = (__bf16)z;
                sZ[t * LXM + u] = hi;
                sZ[QM * LXM + t * LXM + u] = (__bf16)(z - (float)hi);
            }
        }
        const float crt = block_sum<NTH>(cr, s_red);  // also orders the Z stores before the reads below
        if (threadIdx.x == 0) crs[(b * nheads + h) * nch + c] = __expf(tk.cs[QM - 1]) * crt;
        const float tot = tk.cs[QM - 1];
#pragma unroll 1
        for (int k0 = 0; k0 < QM; k0 += 16) {
            const bf16x8 bb = frag_tr(sB, LS, k0, 32 * nt), cc = frag_tr(sC, LS, k0, 32 * nt);
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                const __bf16 *z = sZ + part * QM * LXM;
                accC = mfma_bf16(frag_rm(z, LXM, 32 * mt, k0), bb, accC);
                accB = mfma_bf16(frag_tr(z, LXM, k0, 32 * mt), cc, accB);
            }
        }
        // The states' terms, one direction at a time (dir 0: Hf, Gf with ef; dir 1: Hb, Gb with eb). The A
        // operand's row (token u of dB) is this lane's, so its weight scales the x fragment in registers.
        const int s = 32 * nt + (lane & 31);
#pragma unroll
        for (int dir = 0; dir < 2; ++dir) {
            const float wx = dir ? tk.eb[32 * mt + (lane & 31)] : tk.ef[32 * mt + (lane & 31)];
            const __bf16 *sHd = sH + dir * PM * LS, *sGd = sH + (2 + dir) * PM * LS;
            f32x16 hd = f32x16{};
#pragma unroll 1
            for (int k0 = 0; k0 < PM; k0 += 16) {
                const bf16x8 ya = frag_rm(sY, LXM, 32 * mt, k0), xa = frag_rm(sX, LXM, 32 * mt, k0);
                bf16x8 xw;
#pragma unroll
                for (int j = 0; j < 8; ++j) xw[j] = (__bf16)(wx * (float)xa[j]);
                hd = mfma_bf16(ya, frag_tr(sHd, LS, k0, 32 * nt), hd);
                accB = mfma_bf16(xw, frag_tr(sGd, LS, k0, 32 * nt), accB);
            }
            float pr[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = 32 * mt + acc_row(e, lane);  // token of this row of dC
                const float v = (dir ? __expf(tot - tk.ce[t]) : __expf(tk.cs[t])) * hd[e];
                accC[e] += v;
                pr[e] = (float)sC[t * LS + s] * v;
            }
            const float r = half_sum16(pr);
            if ((lane & 1) == 0) s_rp[(dir * NT + nt) * QM + 32 * mt + acc_row((lane & 31) >> 1, lane)] = r;
        }
        lds_barrier();  // this head's reads of the staged operands are done
        for (int t = threadIdx.x; t < QM; t += NTH) {
            float vf = 0.f, vb = 0.f;
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                vf += s_rp[k * QM + t];
                vb += s_rp[(NT + k) * QM + t];
            }
            rfo[row + t] = vf;
            rbo[row + t] = vb;
        }
        if (hk + 1 < hpg) cr = stage(h + 1);
    }
    const float inv_cnt = R > 0 ? 1.f / (float)(pt * ph * pw) : 0.f;
    const int s = 32 * nt + (lane & 31);
    float rvB[16];  // the review tokens' shares of this wave's dB tile, loaded together
    if (R > 0)
#pragma unroll
        for (int e = 0; e < 16; ++e) rvB[e] = drBg[((b * R + s_rv[32 * mt + acc_row(e, lane)]) * G + g) * S + s];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int t = 32 * mt + acc_row(e, lane);
        const uint32_t n = s_n[t];
        if (n != kNoToken) {
            const size_t o = ((b * N + n) * G + g) * S + s;
            float vb = accB[e];
            if (R > 0) vb += rvB[e] * inv_cnt;
            dB[o] = (__bf16)vb;
            dC[o] = (__bf16)accC[e];
        }
    }
}

// Inclusive prefix (SUFFIX false) or suffix sum over the 64 lanes of a wave.
template <bool SUFFIX>
__device__ __forceinline__ float wave_scan(float v)
{
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = SUFFIX ? __shfl_down(v, off, 64) : __shfl_up(v, off, 64);
        if (SUFFIX ? l + off < 64 : l >= off) v += y;
    }
    return v;
}

// ---------------------------------------------------------------------------
// dx and ddt of one chunk and head on MFMA. CB = C B^T and DX = dy x^T (tile (t, u) per wave) give
// M = CB o L (to LDS as bf16 hi + lo) and, in registers, W = M o DX (t != u), whose strict row and column
// sums are reduced across lanes; then per wave a tile (u, p) of (Gf, Gb read as MFMA operands from memory)
//   dx = M^T dy + ef_u (B Gf^T) + eb_u (B Gb^T) + 2 D dy (+ the review token's share),
// and the per-token sums expl, cf, cb. Last, one wave (a lane per token k) forms
//   span(k) = Sf(k) + sum_{t >= k} rf_t + sum_{u < k} cf_u + Sb(k) + sum_{t <= k} rb_t + sum_{u > k} cb_u
//             + exp(tot) (<Hf, Gf> + <Hb, Gb>)
// (Sf, Sb as in k_bwd_ddt; rf, rb and the cross term from the dB/dC kernel) with two wave scans:
// ddt_k = expl_k + A span(k), and the chunk's parts of dA and dD.
// grid (8 nheads ceil(nch / 8), batch), 256 threads (chunk and head as in chunk_head_of).
// ---------------------------------------------------------------------------
template <int S>
__global__ __launch_bounds__(NTB) void k_bwd_dx_mfma(const __bf16 *__restrict__ x, const __bf16 *__restrict__ dy,
                                                     const __bf16 *__restrict__ Bm, const __bf16 *__restrict__ Cm,
                                                     const float *__restrict__ dtT, const float *__restrict__ csT,
                                                     const float *__restrict__ A, const float *__restrict__ Dv,
                                                     const __bf16 *__restrict__ Gf, const __bf16 *__restrict__ Gb,
                                                     const float *__restrict__ rfi, const float *__restrict__ rbi,
                                                     const float *__restrict__ crs, const float *__restrict__ drx,
                                                     const float *__restrict__ drdt, const int *__restrict__ rinv,
                                                     __bf16 *__restrict__ dx, float *__restrict__ ddt,
                                                     float *__restrict__ pA, float *__restrict__ pD, int nheads, int G,
                                                     uint32_t N, uint32_t Lpad, uint32_t nch, int order, uint32_t T,
                                                     uint32_t H, uint32_t W, int pt, int ph, int pw, uint32_t R)
{
    constexpr int LS = S + 8;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    __shared__ uint32_t s_n[QM], s_rv[QM];
    __bf16 *sB = (__bf16 *)smem_raw;       // [Q][LS]
    __bf16 *sC = sB + QM * LS;             // [Q][LS]
    __bf16 *sX = sC + QM * LS;             // [Q][LXM]
    __bf16 *sY = sX + QM * LXM;            // [Q][LXM]
    __bf16 *sM = sY + QM * LXM;            // 2 x [Q][LXM]  M_tu as bf16 hi + lo
    float *tkm = (float *)(sM + 2 * QM * LXM);
    const TokLds tk{tkm, tkm + QM, tkm + 2 * QM, tkm + 3 * QM, tkm + 4 * QM};
    float *s_red = tkm + 5 * QM;           // [3][2][Q]: expl, cf, cb partials per p-tile
    float *s_w = s_red + 6 * QM;           // [4][2][Q]: W's column sums below / above, row sums left / right
    float *s_blk = s_w + 8 * QM;           // [NTB / 64]
    uint32_t c;
    int h;
    if (!chunk_head_of(nch, nheads, c, h)) return;
    const int g = h / (nheads / G);
    const size_t b = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const size_t row = (b * nheads + h) * Lpad + (size_t)c * QM;
    const size_t PS = (size_t)PM * S, so = ((b * nheads + h) * nch + c) * PS;
    const float a = A[h];
    // the dt tail's inputs from the dB/dC kernel, for wave 0 (a lane per token)
    float rf_k = 0.f, rb_k = 0.f, cr_c = 0.f;
    if (wave == 0) {
        rf_k = rfi[row + lane];
        rb_k = rbi[row + lane];
        cr_c = crs[(b * nheads + h) * nch + c];
    }
    chunk_tokens(s_n, s_rv, c, N, order, T, H, W, rinv, pt, ph, pw, R);
    load_tokens(tk, dtT, csT, row, QM, a);
    lds_barrier();
    // Loads in the order of use (the memory counters retire in order): the chunk's rows, then the B
    // operands of this wave's dx tile straight from the stored states (rows 32 nt + l % 32 of Gf and Gb),
    // then the review tokens' shares of the outputs
    u32x4v rb_rows[QM * S / 8 / NTB], rc_rows[QM * S / 8 / NTB], rx_rows[QM * PM / 8 / NTB],
        ry_rows[QM * PM / 8 / NTB];
    fetch_rows<S, NTB>(rb_rows, Bm, G, g, s_n, b, N);
    fetch_rows<S, NTB>(rc_rows, Cm, G, g, s_n, b, N);
    fetch_rows<PM, NTB>(rx_rows, x, nheads, h, s_n, b, N);
    fetch_rows<PM, NTB>(ry_rows, dy, nheads, h, s_n, b, N);
    bf16x8 gfr[S / 16], gbr[S / 16];
    {
        const size_t o = so + (size_t)(32 * (wave & 1) + (lane & 31)) * S + 8 * (lane >> 5);
#pragma unroll
        for (int k = 0; k < S / 16; ++k) {
            gfr[k] = *(const bf16x8 *)(Gf + o + 16 * k);
            gbr[k] = *(const bf16x8 *)(Gb + o + 16 * k);
        }
    }
    float rvx[16], rvt = 0.f;
    if (R > 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            rvx[e] = drx[((b * R + s_rv[32 * (wave >> 1) + acc_row(e, lane)]) * nheads + h) * PM + 32 * (wave & 1) +
                         (lane & 31)];
        if (wave == 0) rvt = drdt[(b * R + s_rv[lane]) * nheads + h];
    }
    store_rows<S, NTB>(sB, LS, rb_rows, s_n);
    store_rows<S, NTB>(sC, LS, rc_rows, s_n);
    store_rows<PM, NTB>(sX, LXM, rx_rows, s_n);
    store_rows<PM, NTB>(sY, LXM, ry_rows, s_n);
    lds_barrier();
    float xdy = 0.f;  // x . dy over the chunk (rows past the end hold zeros)
    for (int e = threadIdx.x; e < QM * PM; e += NTB) {
        const int u = e / PM, p = e - u * PM;
        xdy += (float)sX[u * LXM + p] * (float)sY[u * LXM + p];
    }
    {  // CB and DX tile (t, u) of this wave: M, and W's strict row and column sums
        const int mt = wave >> 1, nt = wave & 1;
        f32x16 cb = f32x16{}, d = f32x16{};
#pragma unroll
        for (int k0 = 0; k0 < S; k0 += 16)
            cb = mfma_bf16(frag_rm(sC, LS, 32 * mt, k0), frag_rm(sB, LS, 32 * nt, k0), cb);
#pragma unroll
        for (int k0 = 0; k0 < PM; k0 += 16)
            d = mfma_bf16(frag_rm(sY, LXM, 32 * mt, k0), frag_rm(sX, LXM, 32 * nt, k0), d);
        const int u = 32 * nt + (lane & 31);
        float below = 0.f, above = 0.f, left[16], right[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int t = 32 * mt + acc_row(e, lane);
            const float m = cb[e] * ldt_sel(tk, t, u);
            const __bf16 hi = (__bf16)m;
            sM[t * LXM + u] = hi;
            sM[QM * LXM + t * LXM + u] = (__bf16)(m - (float)hi);
            const float w = m * d[e];
            below += t > u ? w : 0.f;
            above += t < u ? w : 0.f;
            left[e] = u < t ? w : 0.f;
            right[e] = u > t ? w : 0.f;
        }
        below += __shfl_xor(below, 32, 64);
        above += __shfl_xor(above, 32, 64);
        const float rl = half_sum16(left), rr = half_sum16(right);
        if (lane < 32) {
            s_w[(0 * 2 + mt) * QM + u] = below;
            s_w[(1 * 2 + mt) * QM + u] = above;
        }
        if ((lane & 1) == 0) {
            const int t = 32 * mt + acc_row((lane & 31) >> 1, lane);
            s_w[(2 * 2 + nt) * QM + t] = rl;
            s_w[(3 * 2 + nt) * QM + t] = rr;
        }
    }
    const float dD = block_sum<NTB>(xdy, s_blk);  // also orders the M stores before the reads below
    {  // dx tile (u, p) of this wave
        const int mt = wave >> 1, nt = wave & 1;
        f32x16 in = f32x16{}, af = f32x16{}, ab = f32x16{};
#pragma unroll
        for (int k0 = 0; k0 < QM; k0 += 16) {
            const bf16x8 yy = frag_tr(sY, LXM, k0, 32 * nt);
            in = mfma_bf16(frag_tr(sM, LXM, k0, 32 * mt), yy, in);
            in = mfma_bf16(frag_tr(sM + QM * LXM, LXM, k0, 32 * mt), yy, in);
        }
#pragma unroll
        for (int k0 = 0; k0 < S; k0 += 16) {
            const bf16x8 ba = frag_rm(sB, LS, 32 * mt, k0);
            af = mfma_bf16(ba, gfr[k0 / 16], af);
            ab = mfma_bf16(ba, gbr[k0 / 16], ab);
        }
        const int p = 32 * nt + (lane & 31);
        const float twoD = 2.f * Dv[h];
        const float inv_cnt = R > 0 ? 1.f / (float)(pt * ph * pw) : 0.f;
        // The dx tile leaves through LDS as 16-byte row pieces: a 32 x 32 staging area per wave in sC,
        // whose last reads (the C B^T tile) precede the barrier of block_sum. Row r sits in slot
        // r ^ ((r >> 2) & 1), so that the two rows one accumulator element writes (r, r + 4) fall on
        // different banks.
        typedef uint32_t piece __attribute__((ext_vector_type(4)));
        static_assert(QM * LS >= NTB / 64 * 32 * 32, "sC holds every wave's staging area");
        __bf16 *stg = sC + wave * (32 * 32);
        auto slot = [](int r) { return r ^ ((r >> 2) & 1); };
        float ve[16], vf[16], vb[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int u = 32 * mt + acc_row(e, lane);
            const float sf = tk.ef[u] * af[e], sb = tk.eb[u] * ab[e];
            const float scan = in[e] + sf + sb;
            const float xv = (float)sX[u * LXM + p], dtu = tk.dt[u];
            ve[e] = dtu > 0.f ? xv * scan / dtu : 0.f;
            vf[e] = xv * sf;
            vb[e] = xv * sb;
            float v = scan + twoD * (float)sY[u * LXM + p];
            if (R > 0) v += rvx[e] * inv_cnt;
            stg[slot(acc_row(e, lane)) * 32 + (lane & 31)] = (__bf16)v;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int idx = lane + 64 * k, rr = idx >> 2, pc = idx & 3;
            const uint32_t n = s_n[32 * mt + rr];
            if (n != kNoToken)
                *(piece *)(dx + ((b * N + n) * nheads + h) * PM + 32 * nt + 8 * pc) =
                    *(const piece *)(stg + slot(rr) * 32 + 8 * pc);
        }
        const float re = half_sum16(ve), rf = half_sum16(vf), rb = half_sum16(vb);
        if ((lane & 1) == 0) {
            const int u = 32 * mt + acc_row((lane & 31) >> 1, lane);
            s_red[(0 * 2 + nt) * QM + u] = re;
            s_red[(1 * 2 + nt) * QM + u] = rf;
            s_red[(2 * 2 + nt) * QM + u] = rb;
        }
    }
    lds_barrier();
    if (wave == 0) {  // lane k: token k of the chunk
        const int k = lane;
        const float expl = s_red[k] + s_red[QM + k];
        const float cf = s_red[2 * QM + k] + s_red[3 * QM + k], cbk = s_red[4 * QM + k] + s_red[5 * QM + k];
        const float dj_f = (s_w[k] + s_w[QM + k]) - (s_w[4 * QM + k] + s_w[5 * QM + k]);
        const float dj_b = (s_w[6 * QM + k] + s_w[7 * QM + k]) - (s_w[2 * QM + k] + s_w[3 * QM + k]);
        // Sf + cf_lt: exclusive prefix of dj_f + cf; Sb + rb_le: inclusive prefix of dj_b + rb;
        // rf_ge: inclusive suffix of rf; cb_gt: exclusive suffix of cb
        const float fa = dj_f + cf;
        const float pre = wave_scan<false>(fa + dj_b + rb_k) - fa;
        const float suf = wave_scan<true>(rf_k + cbk) - cbk;
        const float span = pre + suf + cr_c;
        const uint32_t n = s_n[k];
        float dA = 0.f;
        if (n != kNoToken) {
            float v = expl + a * span;
            if (R > 0) v += rvt / (float)(pt * ph * pw);
            ddt[(b * N + n) * nheads + h] = v;
            dA = tk.dt[k] * span;
        }
        for (int off = 32; off > 0; off >>= 1) dA += __shfl_xor(dA, off, 64);
        if (lane == 0) {
            pA[(b * nheads + h) * nch + c] = dA;
            pD[(b * nheads + h) * nch + c] = 2.f * dD;
        }
    }
}

// LDS bytes of the two MFMA kernels.
template <int S>
constexpr size_t dbdc_mfma_lds()
{
    return (size_t)2 * QM * (S + 8) * 2 + 4 * QM * LXM * 2 + 4 * PM * (S + 8) * 2 +
           (5 * QM + 2 * (S / 32) * QM + 4 * S / 64) * 4;
}
template <int S>
constexpr size_t dx_mfma_lds()
{
    return (size_t)2 * QM * (S + 8) * 2 + 4 * QM * LXM * 2 + (5 * QM + 6 * QM + 8 * QM + NTB / 64) * 4;
}

static_assert(dbdc_mfma_lds<128>() <= 160 * 1024 && dx_mfma_lds<128>() <= 160 * 1024, "LDS of the MFMA kernels");

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// LDS floats of the dB/dC kernel (the largest of the per-chunk kernels) for chunk Q.
size_t dbdc_lds(int Q, int P, int S)
{
    return (size_t)2 * Q * (S + 1) + 2 * Q * (P + 1) + (size_t)Q * (Q + 1) + 4 * P * (SL + 1) + 5 * Q;
}

// The MFMA kernels take bf16 tensors with headdim 64 and d_state 64 or 128.
bool bwd_mfma(const SsdProblem &p) { return p.dtype != 0 && p.headdim == PM && (p.d_state == 64 || p.d_state == 128); }

int bwd_chunk(const SsdProblem &p)
{
    if (bwd_mfma(p)) return QM;
    return dbdc_lds(64, p.headdim, p.d_state) * 4 <= 150 * 1024 ? 64 : 32;
}

struct BwdLayout {
    int Q, nch, nchR;
    size_t dtT, csT, Sf, Sb, Uf, Ub, CB, expl, cf, cb, rf, rb, crs, pA, pD;
    size_t rx, rB, rdt, rdtT, rcsT, rSf, rSb, h0f, h0b, Gf0, Gb0, drx, drB, drBg, drdt, pAr, rcf, rcb, rinv, total;
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
    const size_t se = bwd_mfma(p) ? 2 : 4;  // bytes per stored state element (bf16 on the MFMA path)
    l.Sf = take(B * Hs * l.nch * PS * se);
    l.Sb = take(B * Hs * l.nch * PS * se);
    l.Uf = take(B * Hs * l.nch * PS * se);
    l.Ub = take(B * Hs * l.nch * PS * se);
    if (bwd_mfma(p)) {
        l.crs = take(B * Hs * l.nch * 4);
    } else {
        l.CB = take(B * G * l.nch * (size_t)l.Q * l.Q * 4);
        l.expl = take(B * Hs * Lpad * 4);
        l.cf = take(B * Hs * Lpad * 4);
        l.cb = take(B * Hs * Lpad * 4);
    }
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
        l.rcf = take(B * Hs * R * 4);
        l.rcb = take(B * Hs * R * 4);
        l.rinv = take(R * 4);
    }
    l.total = off;
    return l;
}

size_t review_lds(const SsdProblem &p)
{
    return ((size_t)2 * p.headdim * p.d_state + p.headdim + p.d_state + 2 * RT + 2 * NTB) * 4;
}

// Chunk states, their passes, and the per-chunk gradient kernels on MFMA (after the review tokens'
// states and dt's cumulative sums are in place).
template <int S>
hipError_t run_chunks_mfma(const SsdProblem &p, const SsdGradArgs &a, const BwdLayout &l, char *w, const int *rinv,
                           const float *h0f, const float *h0b, float *Gf0, float *Gb0, const float *drx,
                           const float *drdt, const float *drBg, const float *pAr, hipStream_t st)
{
    auto F = [&](size_t off) { return (float *)(w + off); };
    auto Hh = [&](size_t off) { return (__bf16 *)(w + off); };
    float *dtT = F(l.dtT), *csT = F(l.csT);
    __bf16 *Sf = Hh(l.Sf), *Sb = Hh(l.Sb), *Uf = Hh(l.Uf), *Ub = Hh(l.Ub);
    float *rf = F(l.rf), *rb = F(l.rb), *crs = F(l.crs), *pA = F(l.pA), *pD = F(l.pD);
    const int Hs = p.nheads, G = p.ngroups, B = (int)p.batch;
    const uint32_t N = (uint32_t)p.N, Lpad = (uint32_t)(l.nch * QM), R = (uint32_t)p.R;
    const uint32_t T = (uint32_t)p.T, H = (uint32_t)p.H, W = (uint32_t)p.W;
    const __bf16 *x = (const __bf16 *)a.x, *Bm = (const __bf16 *)a.b, *Cm = (const __bf16 *)a.c;
    const __bf16 *dy = (const __bf16 *)a.dy;
    const uint32_t nch = (uint32_t)l.nch;
    const dim3 gh(8 * Hs * ((nch + 7) / 8), B), gg(nch, G, B), gp((PM * S / 8 + 255) / 256, 2 * Hs, B);
    k_bwd_states_mfma<S, false><<<gh, NTB, 0, st>>>(x, Bm, dtT, csT, a.a, Sf, Sb, Hs, G, N, Lpad, nch, p.order, T, H,
                                                    W);
    k_state_pass_bf16<<<gp, 256, 0, st>>>(Sf, Sb, csT, h0f, h0b, nullptr, nullptr, PM * S, l.nch, Lpad);
    k_bwd_states_mfma<S, true><<<gh, NTB, 0, st>>>(dy, Cm, dtT, csT, a.a, Uf, Ub, Hs, G, N, Lpad, nch, p.order, T, H,
                                                   W);
    k_state_pass_bf16<<<gp, 256, 0, st>>>(Ub, Uf, csT, nullptr, nullptr, Gb0, Gf0, PM * S, l.nch, Lpad);
    if (R > 0) {
        k_review_grads<<<((R + RT - 1) / RT) * B * Hs, NTB, review_lds(p), st>>>(
            F(l.rx), F(l.rB), F(l.rdt), a.a, Gf0, Gb0, (float *)drx, F(l.drB), (float *)drdt, F(l.rcf), F(l.rcb), Hs,
            PM, S, G, (int)R);
        k_review_spans<<<(B * Hs + 255) / 256, 256, 0, st>>>(F(l.rdt), a.a, F(l.rcf), F(l.rcb), (float *)drdt,
                                                            (float *)pAr, Hs, (int)R, B * Hs);
        k_review_group<<<dim3(R, B), 256, 0, st>>>(F(l.drB), (float *)drBg, Hs, S, G);
    }
    k_bwd_dbdc_mfma<S><<<gg, 4 * S, dbdc_mfma_lds<S>(), st>>>(
        x, dy, Bm, Cm, dtT, csT, a.a, Sf, Sb, Uf, Ub, drBg, rinv, (__bf16 *)a.db, (__bf16 *)a.dc, rf, rb, crs, Hs, G,
        N, Lpad, p.order, T, H, W, p.pool_t, p.pool_h, p.pool_w, R);
    k_bwd_dx_mfma<S><<<gh, NTB, dx_mfma_lds<S>(), st>>>(x, dy, Bm, Cm, dtT, csT, a.a, a.d, Uf, Ub, rf, rb, crs, drx,
                                                        drdt, rinv, (__bf16 *)a.dx, a.ddt, pA, pD, Hs, G, N, Lpad,
                                                        nch, p.order, T, H, W, p.pool_t, p.pool_h, p.pool_w, R);
    k_bwd_reduce<<<(Hs + 255) / 256, 256, 0, st>>>(pA, pD, pAr, a.da, a.dd, Hs, l.nch, B);
    return hipGetLastError();
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
        // bf16 rows of a multiple of 8 channels pool 8 channels per thread, fp32 rows of a multiple of 4
        // (16-byte aligned) 4 per thread; anything else one channel per thread
        auto pool_rows = [&](const E *src, float *dst, int64_t C) {
            if constexpr (std::is_same<E, bf16_t>::value) {
                if (C % 8 == 0 && ((uintptr_t)src & 15) == 0) {
                    ssd::k_pool8<float><<<dim3((unsigned)((C + 2047) / 2048), R, B), 256, 0, st>>>(
                        src, dst, C, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
                    return;
                }
            }
            k_pool<E, float><<<dim3((unsigned)((C + 255) / 256), R, B), 256, 0, st>>>(src, dst, C, T, H, W, p.pool_t,
                                                                                    p.pool_h, p.pool_w, p.order);
        };
        pool_rows(x, rx, Cx);
        pool_rows(Bm, rB, Cbw);
        if (ssd::pool_f32x4_ok(a.dt, Hs))
            ssd::k_pool_f32x4<<<dim3(R, B), ssd::kPoolF4Threads, 0, st>>>(a.dt, rdt, Hs, T, H, W, p.pool_t, p.pool_h, p.pool_w,
                                                         p.order);
        else
            k_pool<float, float><<<dim3((Hs + 255) / 256, R, B), 256, 0, st>>>(a.dt, rdt, Hs, T, H, W, p.pool_t,
                                                                              p.pool_h, p.pool_w, p.order);
        prep_dt<false>(rdt, a.a, rdtT, rcsT, Hs, R, Rpad, Q, 0, 1, 1, R, l.nchR, B, st);
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
    prep_dt<true>(a.dt, a.a, dtT, csT, Hs, N, Lpad, Q, p.order, T, H, W, l.nch, B, st);
    if constexpr (std::is_same<E, bf16_t>::value) {
        if (bwd_mfma(p)) {
            if (S == 64) return run_chunks_mfma<64>(p, a, l, w, rinv, h0f, h0b, Gf0, Gb0, drx, drdt, drBg, pAr, st);
            return run_chunks_mfma<128>(p, a, l, w, rinv, h0f, h0b, Gf0, Gb0, drx, drdt, drBg, pAr, st);
        }
    }
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
        k_review_grads<<<((R + RT - 1) / RT) * B * Hs, NTB, review_lds(p), st>>>(
            F(l.rx), F(l.rB), F(l.rdt), a.a, Gf0, Gb0, drx, F(l.drB), drdt, F(l.rcf), F(l.rcb), Hs, P, S, G, (int)R);
        k_review_spans<<<(B * Hs + 255) / 256, 256, 0, st>>>(F(l.rdt), a.a, F(l.rcf), F(l.rcb), drdt, pAr, Hs,
                                                            (int)R, B * Hs);
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
    // the review-token gradient launch: a workgroup per RT review tokens, head and batch element, its
    // work-items below 2^32
    const int64_t review_groups = (p.R + RT - 1) / RT * p.batch * p.nheads;
    return (p.headdim == 16 || p.headdim == 32 || p.headdim == 64) && p.d_state <= 128 && p.d_state % 8 == 0 &&
           (size_t)review_lds(p) <= 160 * 1024 && review_groups * NTB < ((int64_t)1 << 32);
}

size_t ssd_backward_workspace(const SsdProblem &p) { return bwd_layout(p).total; }

hipError_t ssd_backward_prepare()
{
    hipError_t e;
    if ((e = set_lds_attrs<float>()) != hipSuccess) return e;
    if ((e = set_lds_attrs<bf16_t>()) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_chunk_states<float, false, false>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024)) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_bwd_dbdc_mfma<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)dbdc_mfma_lds<64>())) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_bwd_dbdc_mfma<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)dbdc_mfma_lds<128>())) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_bwd_dx_mfma<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)dx_mfma_lds<64>())) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_bwd_dx_mfma<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)dx_mfma_lds<128>())) != hipSuccess) return e;
    return hipFuncSetAttribute((const void *)k_review_grads, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

hipError_t ssd_backward(const SsdProblem &p, const SsdGradArgs &a, void *ws, hipStream_t st)
{
    if (p.dtype == 0) return run_backward<float>(p, a, ws, st);
    return run_backward<bf16_t>(p, a, ws, st);
}

} // namespace mate
