// Portable chunked evaluation of the bidirectional Mamba2 scan (fp32 FMA, any
// supported head size). It is the path for fp32 tensors and for shapes the
// MFMA kernels are not built for.
//
// The recurrence h_u = exp(a_u) h_{u-1} + dt_u x_u B_u^T, y_u = h_u C_u + D x_u
// (a_u = dt_u A) is evaluated in chunks of Q tokens (the Mamba2 "state space
// duality" split that the xllm-io review of LinGen, section 三 item 1, refers
// to). With cs_t the inclusive cumulative sum of a inside a chunk,
// ce_t = cs_t - a_t and tot = cs_{Q-1}, the sum of both directions is
//   y_t = sum_u (C_t . B_u) dt_u w(t,u) x_u                         (intra chunk)
//       + exp(cs_t) Hf C_t + exp(tot - ce_t) Hb C_t                  (inter chunk)
//       + 2 D x_t
// with w = exp(cs_t - cs_u) below the diagonal, exp(ce_u - ce_t) above it and
// 2 on it; Hf is the forward state entering the chunk from the left and Hb the
// backward state entering it from the right. Chunk contributions to the states:
//   Sf = sum_u exp(tot - cs_u) dt_u x_u B_u^T,  Sb = sum_u exp(ce_u) dt_u x_u B_u^T,
// and across a chunk both states decay by exp(tot).
#include "common.hpp"
#include "launch.hpp"
#include "ssd_chunks.hpp"
#include "ssd_common.hpp"
#include "timing.hpp"

namespace mate {

namespace {

using ssd::kMaxQ;
using ssd::k_cb;
using ssd::k_chunk_states;
using ssd::k_state_pass;
using ssd::k_pool;
using ssd::prep_dt;
using ssd::k_pool_f32x4;
using ssd::pool_f32x4_ok;
using ssd::seq_row;


// Outputs of one chunk and head; Sf / Sb hold the entering states.
// grid (nchunks, nheads, batch), 256 threads.
template <typename E>
__global__ __launch_bounds__(256) void k_output(const E *__restrict__ x, const E *__restrict__ Cm,
                                                const float *__restrict__ CB, const float *__restrict__ dtT,
                                                const float *__restrict__ csT, const float *__restrict__ A,
                                                const float *__restrict__ Dv, const float *__restrict__ Hf,
                                                const float *__restrict__ Hb, E *__restrict__ y, int nheads, int P,
                                                int S, int G, uint32_t N, uint32_t Lpad, int Q, int order,
                                                uint32_t T_, uint32_t H, uint32_t W)
{
    constexpr int kMaxOut = kMaxQ * 128 / 256;  // Q * P / 256 outputs per thread at most
    __shared__ float sm[kMaxQ * (kMaxQ + 1) + kMaxQ * 129];
    __shared__ float s_dt[kMaxQ], s_cs[kMaxQ];
    const uint32_t c = blockIdx.x, b = blockIdx.z, nch = gridDim.x;
    const int h = blockIdx.y, g = h / (nheads / G);
    const int QP = Q * P, PS = P * S;
    const size_t row = ((size_t)b * nheads + h) * Lpad + (size_t)c * Q;
    const float a = A[h];
    const float tot = csT[row + Q - 1];
    for (int u = threadIdx.x; u < Q; u += 256) {
        s_dt[u] = dtT[row + u];
        s_cs[u] = csT[row + u];
    }
    const float *hf = Hf + (((size_t)b * nheads + h) * nch + c) * PS;
    const float *hb = Hb + (((size_t)b * nheads + h) * nch + c) * PS;

    // Phase 1: inter-chunk terms. LDS: Hf, Hb (P x 33) and C (Q x 33) per 32-wide slice of S.
    float *sHf = sm, *sHb = sm + P * 33, *sC = sm + 2 * P * 33;
    float accf[kMaxOut], accb[kMaxOut];
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) accf[k] = accb[k] = 0.f;
    for (int s0 = 0; s0 < S; s0 += 32) {
        __syncthreads();
        for (int k = threadIdx.x; k < P * 32; k += 256) {
            const int p = k >> 5, s = k & 31;
            const bool ok = s0 + s < S;
            sHf[p * 33 + s] = ok ? hf[p * S + s0 + s] : 0.f;
            sHb[p * 33 + s] = ok ? hb[p * S + s0 + s] : 0.f;
        }
        for (int k = threadIdx.x; k < Q * 32; k += 256) {
            const int u = k >> 5, s = k & 31;
            const uint32_t i = c * Q + u;
            float v = 0.f;
            if (i < N && s0 + s < S)
                v = elem<E>::load(Cm + (((size_t)b * N + rms_index32(i, order, T_, H, W)) * G + g) * S + s0 + s);
            sC[u * 33 + s] = v;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k) {
            const int e = threadIdx.x + 256 * k;
            if (e < QP) {
                const int t = e / P, p = e - t * P;
                float af = 0.f, ab = 0.f;
                for (int s = 0; s < 32; ++s) {
                    const float cv = sC[t * 33 + s];
                    af += sHf[p * 33 + s] * cv;
                    ab += sHb[p * 33 + s] * cv;
                }
                accf[k] += af;
                accb[k] += ab;
            }
        }
    }
    __syncthreads();

    // Phase 2: intra-chunk term. LDS: weighted CB (Q x Q+1) and X (Q x P+1).
    float *sM = sm, *sX = sm + Q * (Q + 1);
    const float *cb = CB + (((size_t)b * G + g) * nch + c) * Q * Q;
    for (int k = threadIdx.x; k < Q * Q; k += 256) {
        const int t = k / Q, u = k - t * Q;
        float w;
        if (u < t)
            w = __expf(s_cs[t] - s_cs[u]);
        else if (u > t)
            w = __expf((s_cs[u] - s_dt[u] * a) - (s_cs[t] - s_dt[t] * a));
        else
            w = 2.f;
        sM[t * (Q + 1) + u] = cb[k] * s_dt[u] * w;
    }
    for (int k = threadIdx.x; k < Q * P; k += 256) {
        const int u = k / P, p = k - u * P;
        const uint32_t i = c * Q + u;
        float v = 0.f;
        if (i < N) v = elem<E>::load(x + (((size_t)b * N + rms_index32(i, order, T_, H, W)) * nheads + h) * P + p);
        sX[u * (P + 1) + p] = v;
    }
    __syncthreads();
    const float two_d = 2.f * Dv[h];
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) {
        const int e = threadIdx.x + 256 * k;
        if (e < QP) {
            const int t = e / P, p = e - t * P;
            const uint32_t i = c * Q + t;
            float acc = __expf(s_cs[t]) * accf[k] + __expf(tot - (s_cs[t] - s_dt[t] * a)) * accb[k];
            for (int u = 0; u < Q; ++u) acc += sM[t * (Q + 1) + u] * sX[u * (P + 1) + p];
            acc += two_d * sX[t * (P + 1) + p];
            if (i < N)
                elem<E>::store(y + (((size_t)b * N + rms_index32(i, order, T_, H, W)) * nheads + h) * P + p, acc);
        }
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

} // namespace

// Workspace carve-up of the portable path (all fp32):
//   dtT, csT      [batch][nheads][Lpad]            main sequence
//   Sf, Sb        [batch][nheads][nch][P][S]       chunk states, then entering states
//   CB            [batch][G][nch][Q][Q]
//   review only:  rx [batch][R][nheads][P], rB [batch][R][G][S], rdt [batch][R][nheads],
//                 rdtT, rcsT [batch][nheads][Rpad], rSf, rSb [batch][nheads][nchR][P][S],
//                 h0f, h0b [batch][nheads][P][S]
struct PortableLayout {
    size_t dtT, csT, Sf, Sb, CB, rx, rB, rdt, rdtT, rcsT, rSf, rSb, h0f, h0b, total;
};

static PortableLayout portable_layout(const SsdProblem &p)
{
    PortableLayout l{};
    const size_t B = p.batch, Hs = p.nheads, PS = (size_t)p.headdim * p.d_state;
    const size_t Lpad = (size_t)p.nch * p.chunk;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    l.dtT = take(B * Hs * Lpad * 4);
    l.csT = take(B * Hs * Lpad * 4);
    l.Sf = take(B * Hs * p.nch * PS * 4);
    l.Sb = take(B * Hs * p.nch * PS * 4);
    l.CB = take(B * p.ngroups * p.nch * (size_t)p.chunk * p.chunk * 4);
    if (p.R > 0) {
        const size_t Rpad = (size_t)p.nchR * p.chunk;
        l.rx = take(B * p.R * Hs * p.headdim * 4);
        l.rB = take(B * p.R * p.ngroups * p.d_state * 4);
        l.rdt = take(B * p.R * Hs * 4);
        l.rdtT = take(B * Hs * Rpad * 4);
        l.rcsT = take(B * Hs * Rpad * 4);
        l.rSf = take(B * Hs * p.nchR * PS * 4);
        l.rSb = take(B * Hs * p.nchR * PS * 4);
        l.h0f = take(B * Hs * PS * 4);
        l.h0b = take(B * Hs * PS * 4);
    }
    l.total = off;
    return l;
}

size_t ssd_portable_workspace(const SsdProblem &p) { return portable_layout(p).total; }

template <typename E>
static hipError_t run_portable(const SsdProblem &p, const SsdArgs &a, void *ws, hipStream_t st)
{
    const PortableLayout l = portable_layout(p);
    char *w = (char *)ws;
    float *dtT = (float *)(w + l.dtT), *csT = (float *)(w + l.csT);
    float *Sf = (float *)(w + l.Sf), *Sb = (float *)(w + l.Sb), *CB = (float *)(w + l.CB);
    const int Hs = p.nheads, P = p.headdim, S = p.d_state, G = p.ngroups, Q = p.chunk;
    const uint32_t N = (uint32_t)p.N, Lpad = (uint32_t)(p.nch * Q);
    const uint32_t T = (uint32_t)p.T, H = (uint32_t)p.H, W = (uint32_t)p.W;
    const int B = (int)p.batch;
    const E *x = (const E *)a.x, *Bm = (const E *)a.b, *Cm = (const E *)a.c;
    const size_t states_lds = ((size_t)Q * P + (size_t)Q * S + 2 * Q) * 4;
    hipError_t e;

    float *h0f = nullptr, *h0b = nullptr;
    if (p.R > 0) {
        float *rx = (float *)(w + l.rx), *rB = (float *)(w + l.rB), *rdt = (float *)(w + l.rdt);
        float *rdtT = (float *)(w + l.rdtT), *rcsT = (float *)(w + l.rcsT);
        float *rSf = (float *)(w + l.rSf), *rSb = (float *)(w + l.rSb);
        h0f = (float *)(w + l.h0f);
        h0b = (float *)(w + l.h0b);
        const uint32_t R = (uint32_t)p.R, Rpad = (uint32_t)(p.nchR * Q);
        const int64_t Cx = (int64_t)Hs * P, Cb = (int64_t)G * S;
        {
            timing::Scope ts_(K_SSD_POOL, st);
            k_pool<E, float><<<dim3((Cx + 255) / 256, R, B), 256, 0, st>>>(x, rx, Cx, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        }
        {
            timing::Scope ts_(K_SSD_POOL, st);
            k_pool<E, float><<<dim3((Cb + 255) / 256, R, B), 256, 0, st>>>(Bm, rB, Cb, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        }
        {
            timing::Scope ts_(K_SSD_POOL, st);
            if (pool_f32x4_ok(a.dt, Hs))
                k_pool_f32x4<<<dim3(R, B), ssd::kPoolF4Threads, 0, st>>>(a.dt, rdt, Hs, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
            else
                k_pool<float, float><<<dim3((Hs + 255) / 256, R, B), 256, 0, st>>>(a.dt, rdt, Hs, T, H, W, p.pool_t,
                                                                                  p.pool_h, p.pool_w, p.order);
        }
        {
            timing::Scope ts_(K_SSD_PREP, st);
            prep_dt<false>(rdt, a.a, rdtT, rcsT, Hs, R, Rpad, Q, 0, 1, 1, R, p.nchR, B, st);
        }
        {
            timing::Scope ts_(K_SSD_STATES, st);
            k_chunk_states<float, false, false><<<dim3(p.nchR, Hs, B), 256, states_lds, st>>>(
                rx, rB, rdtT, rcsT, a.a, rSf, rSb, Hs, P, S, G, R, Rpad, Q, 0, 1, 1, R);
        }
        {
            timing::Scope ts_(K_SSD_SEG_PASS, st);
            k_state_pass<<<dim3((P * S + 255) / 256, Hs, B), 256, 0, st>>>(rSf, rSb, rcsT, nullptr, nullptr, h0f, h0b,
                                                                          P * S, p.nchR, Q, Rpad);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        timing::Scope ts_(K_SSD_PREP, st);
        prep_dt<true>(a.dt, a.a, dtT, csT, Hs, N, Lpad, Q, p.order, T, H, W, p.nch, B, st);
    }
    {
        timing::Scope ts_(K_SSD_STATES, st);
        k_chunk_states<E, true, false><<<dim3(p.nch, Hs, B), 256, states_lds, st>>>(x, Bm, dtT, csT, a.a, Sf, Sb, Hs, P, S, G, N,
                                                                             Lpad, Q, p.order, T, H, W);
    }
    {
        timing::Scope ts_(K_SSD_SEG_PASS, st);
        k_state_pass<<<dim3((P * S + 255) / 256, Hs, B), 256, 0, st>>>(Sf, Sb, csT, h0f, h0b, nullptr, nullptr, P * S,
                                                                      p.nch, Q, Lpad);
    }
    {
        timing::Scope ts_(K_SSD_CB, st);
        k_cb<E><<<dim3(p.nch, G, B), 256, 0, st>>>(Bm, Cm, CB, G, S, N, Q, p.order, T, H, W);
    }
    {
        timing::Scope ts_(K_SSD_OUT, st);
        k_output<E><<<dim3(p.nch, Hs, B), 256, 0, st>>>(x, Cm, CB, dtT, csT, a.a, a.d, Sf, Sb, (E *)a.y, Hs, P, S, G, N,
                                                        Lpad, Q, p.order, T, H, W);
    }
    return hipGetLastError();
}

hipError_t ssd_portable(const SsdProblem &p, const SsdArgs &a, void *ws, hipStream_t st)
{
    if (p.dtype == 0) return run_portable<float>(p, a, ws, st);
    return run_portable<bf16_t>(p, a, ws, st);
}

hipError_t ssd_portable_prepare()
{
    // The state kernel may take more than 64 KB of dynamic LDS.
    const int lds = 160 * 1024;
    hipError_t e;
    if ((e = hipFuncSetAttribute((const void *)k_chunk_states<float, false, false>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)k_chunk_states<float, true, false>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess) return e;
    return hipFuncSetAttribute((const void *)k_chunk_states<bf16_t, true, false>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

} // namespace mate
