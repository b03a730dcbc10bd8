// Chunk-level kernels of the portable scan and of the scan's backward: the
// per-chunk state contributions, the pass that turns them into the states
// entering each chunk, and C . B per chunk (all fp32).
#pragma once

#include "common.hpp"
#include "ssd_common.hpp"

namespace mate {
namespace ssd {
namespace {

// Per-chunk state contributions Sf, Sb (P x S, fp32) of one head:
//   Sf = sum_u wf_u x_u B_u^T,  Sb = sum_u wb_u x_u B_u^T
// with wf = dt exp(tot - cs), wb = dt exp(ce) for the states of the scan, or (ADJ, for the adjoint states
// of its backward, x = dy and B = C) wf = exp(cs), wb = exp(tot - ce).
// grid (nchunks, nheads, batch), 256 threads. LDS: X (Q x P) and B (Q x S) in fp32.
template <typename E, bool PERM, bool ADJ>
__global__ __launch_bounds__(256) void k_chunk_states(const E *__restrict__ x, const E *__restrict__ Bm,
                                                      const float *__restrict__ dtT, const float *__restrict__ csT,
                                                      const float *__restrict__ A, float *__restrict__ Sf,
                                                      float *__restrict__ Sb, int nheads, int P, int S, int G,
                                                      uint32_t L, uint32_t Lpad, int Q, int order, uint32_t T,
                                                      uint32_t H, uint32_t W)
{
    extern __shared__ float smem[];
    float *Xs = smem;                 // [Q][P]
    float *Bs = Xs + Q * P;           // [Q][S]
    float *wf = Bs + Q * S;           // [Q]
    float *wb = wf + Q;               // [Q]
    const uint32_t c = blockIdx.x, b = blockIdx.z;
    const int h = blockIdx.y, g = h / (nheads / G);
    const uint32_t nch = gridDim.x;
    for (int k = threadIdx.x; k < Q * P; k += 256) {
        const int u = k / P, p = k - u * P;
        const uint32_t i = c * Q + u;
        float v = 0.f;
        if (i < L) v = elem<E>::load(x + (((size_t)b * L + seq_row<PERM>(i, order, T, H, W)) * nheads + h) * P + p);
        Xs[k] = v;
    }
    for (int k = threadIdx.x; k < Q * S; k += 256) {
        const int u = k / S, s = k - u * S;
        const uint32_t i = c * Q + u;
        float v = 0.f;
        if (i < L) v = elem<E>::load(Bm + (((size_t)b * L + seq_row<PERM>(i, order, T, H, W)) * G + g) * S + s);
        Bs[k] = v;
    }
    const size_t row = ((size_t)b * nheads + h) * Lpad + (size_t)c * Q;
    const float a = A[h];
    const float tot = csT[row + Q - 1];
    for (int u = threadIdx.x; u < Q; u += 256) {
        const float d = dtT[row + u], cs = csT[row + u];
        if (ADJ) {
            wf[u] = __expf(cs);
            wb[u] = __expf(tot - (cs - d * a));
        } else {
            wf[u] = d * __expf(tot - cs);
            wb[u] = d * __expf(cs - d * a);
        }
    }
    __syncthreads();
    const int PS = P * S;
    float *outf = Sf + (((size_t)b * nheads + h) * nch + c) * PS;
    float *outb = Sb + (((size_t)b * nheads + h) * nch + c) * PS;
    for (int e = threadIdx.x; e < PS; e += 256) {
        const int p = e / S, s = e - p * S;
        float af = 0.f, ab = 0.f;
        for (int u = 0; u < Q; ++u) {
            const float xb = Xs[u * P + p] * Bs[u * S + s];
            af += xb * wf[u];
            ab += xb * wb[u];
        }
        outf[e] = af;
        outb[e] = ab;
    }
}

// Turns chunk contributions into the states entering each chunk: Sf[c] becomes
// the forward state after chunk c-1, Sb[c] the backward state after chunk c+1.
// h0f / h0b (optional) are the initial states; finF / finB (optional) receive
// the final states. grid (ceil(P*S / 256), nheads, batch).
__global__ __launch_bounds__(256) void k_state_pass(float *__restrict__ Sf, float *__restrict__ Sb,
                                                    const float *__restrict__ csT, const float *__restrict__ h0f,
                                                    const float *__restrict__ h0b, float *__restrict__ finF,
                                                    float *__restrict__ finB, int PS, int nch, int Q, uint32_t Lpad)
{
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= PS) return;
    const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
    const float *cs = csT + bh * Lpad;
    float *f = Sf + bh * nch * PS + e;
    float *bk = Sb + bh * nch * PS + e;
    float run = h0f ? h0f[bh * PS + e] : 0.f;
    for (int c = 0; c < nch; ++c) {
        const float tot = cs[(size_t)c * Q + Q - 1];
        const float s = f[(size_t)c * PS];
        f[(size_t)c * PS] = run;
        run = __expf(tot) * run + s;
    }
    if (finF) finF[bh * PS + e] = run;
    run = h0b ? h0b[bh * PS + e] : 0.f;
    for (int c = nch - 1; c >= 0; --c) {
        const float tot = cs[(size_t)c * Q + Q - 1];
        const float s = bk[(size_t)c * PS];
        bk[(size_t)c * PS] = run;
        run = __expf(tot) * run + s;
    }
    if (finB) finB[bh * PS + e] = run;
}

// CB[t][u] = C_t . B_u for every chunk and group. grid (nchunks, G, batch).
template <typename E>
__global__ __launch_bounds__(256) void k_cb(const E *__restrict__ Bm, const E *__restrict__ Cm,
                                            float *__restrict__ CB, int G, int S, uint32_t L, int Q, int order,
                                            uint32_t T_, uint32_t H, uint32_t W)
{
    __shared__ float Bs[kMaxQ][33];
    __shared__ float Cs[kMaxQ][33];
    const uint32_t c = blockIdx.x, b = blockIdx.z;
    const int g = blockIdx.y;
    const int QQ = Q * Q;
    float acc[kMaxQ * kMaxQ / 256];
#pragma unroll
    for (int k = 0; k < kMaxQ * kMaxQ / 256; ++k) acc[k] = 0.f;
    for (int s0 = 0; s0 < S; s0 += 32) {
        __syncthreads();
        for (int k = threadIdx.x; k < Q * 32; k += 256) {
            const int u = k >> 5, s = k & 31;
            const uint32_t i = c * Q + u;
            float bv = 0.f, cv = 0.f;
            if (i < L && s0 + s < S) {
                const size_t off = (((size_t)b * L + rms_index32(i, order, T_, H, W)) * G + g) * S + s0 + s;
                bv = elem<E>::load(Bm + off);
                cv = elem<E>::load(Cm + off);
            }
            Bs[u][s] = bv;
            Cs[u][s] = cv;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMaxQ * kMaxQ / 256; ++k) {
            const int e = threadIdx.x + 256 * k;
            if (e < QQ) {
                const int t = e / Q, u = e - t * Q;
                float a = 0.f;
                for (int s = 0; s < 32; ++s) a += Cs[t][s] * Bs[u][s];
                acc[k] += a;
            }
        }
    }
    float *out = CB + (((size_t)b * G + g) * gridDim.x + c) * QQ;
#pragma unroll
    for (int k = 0; k < kMaxQ * kMaxQ / 256; ++k) {
        const int e = threadIdx.x + 256 * k;
        if (e < QQ) out[e] = acc[k];
    }
}

} // namespace
} // namespace ssd
} // namespace mate
