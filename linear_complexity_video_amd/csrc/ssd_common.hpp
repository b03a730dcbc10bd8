// Kernels shared by both evaluations of the bidirectional scan: dt in scan
// order with its per-chunk cumulative sums, and review-token pooling.
#pragma once

#include "common.hpp"

namespace mate {
namespace ssd {

constexpr int kMaxQ = 128;

// Row index of scan position i: the RMS permutation for the main sequence, the
// identity for the (already ordered) review sequence.
template <bool PERM>
__device__ __forceinline__ uint32_t seq_row(uint32_t i, int order, uint32_t T, uint32_t H, uint32_t W)
{
    return PERM ? rms_index32(i, order, T, H, W) : i;
}

// dt in scan order, one row per head, and its within-chunk inclusive cumsum of
// dt * A. Positions >= L are zero (exact no-ops of the recurrence).
// grid (nchunks, ceil(nheads / 64), batch), 256 threads.
template <bool PERM>
__global__ __launch_bounds__(256) void k_prep_dt(const float *__restrict__ dt, const float *__restrict__ A,
                                                 float *__restrict__ dtT, float *__restrict__ csT, int nheads,
                                                 uint32_t L, uint32_t Lpad, int Q, int order, uint32_t T,
                                                 uint32_t H, uint32_t W)
{
    __shared__ float sdt[kMaxQ][65];
    __shared__ float scs[kMaxQ][65];
    const uint32_t c = blockIdx.x, b = blockIdx.z;
    const int h0 = blockIdx.y * 64;
    for (int k = threadIdx.x; k < Q * 64; k += 256) {
        const int u = k >> 6, hh = k & 63, h = h0 + hh;
        const uint32_t i = c * Q + u;
        float v = 0.f;
        if (i < L && h < nheads) v = dt[((size_t)b * L + seq_row<PERM>(i, order, T, H, W)) * nheads + h];
        sdt[u][hh] = v;
    }
    __syncthreads();
    if (threadIdx.x < 64 && h0 + (int)threadIdx.x < nheads) {
        const float a = A[h0 + threadIdx.x];
        float cs = 0.f;
        for (int u = 0; u < Q; ++u) {
            cs += sdt[u][threadIdx.x] * a;
            scs[u][threadIdx.x] = cs;
        }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < Q * 64; k += 256) {
        const int hh = k / Q, u = k - hh * Q, h = h0 + hh;
        if (h >= nheads) continue;
        const size_t o = ((size_t)b * nheads + h) * Lpad + (size_t)c * Q + u;
        dtT[o] = sdt[u][hh];
        csT[o] = scs[u][hh];
    }
}

// Average pool over disjoint pt x ph x pw blocks; out[b][j][ch] with j in RMS
// order `order` of the pooled grid. grid (ceil(C / 256), R, batch).
template <typename E, typename O>
__global__ __launch_bounds__(256) void k_pool(const E *__restrict__ src, O *__restrict__ out, int64_t C,
                                              uint32_t Tn, uint32_t Hn, uint32_t Wn, int pt, int ph, int pw,
                                              int order)
{
    const int64_t ch = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (ch >= C) return;
    const uint32_t j = blockIdx.y, b = blockIdx.z, R = gridDim.y;
    const uint32_t Tp = Tn / pt, Hp = Hn / ph, Wp = Wn / pw;
    const uint32_t np = rms_index32(j, order, Tp, Hp, Wp);
    const uint32_t tq = np / (Hp * Wp), hq = (np / Wp) % Hp, wq = np % Wp;
    const size_t N = (size_t)Tn * Hn * Wn;
    float acc = 0.f;
    for (int dt_ = 0; dt_ < pt; ++dt_)
        for (int dh = 0; dh < ph; ++dh)
            for (int dw = 0; dw < pw; ++dw) {
                const size_t n = ((size_t)(tq * pt + dt_) * Hn + hq * ph + dh) * Wn + wq * pw + dw;
                acc += elem<E>::load(src + ((size_t)b * N + n) * C + ch);
            }
    elem<O>::store(out + ((size_t)b * R + j) * C + ch, acc / (float)(pt * ph * pw));
}

// The same average pool on bf16 input, 8 channels (one 16-byte load) per
// thread; C must be a multiple of 8. Output bf16 (rounded) or fp32.
// grid (ceil(C / 2048), R, batch).
template <typename O>
__global__ __launch_bounds__(256) void k_pool8(const bf16_t *__restrict__ src, O *__restrict__ out, int64_t C,
                                               uint32_t Tn, uint32_t Hn, uint32_t Wn, int pt, int ph, int pw,
                                               int order)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int64_t ch = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (ch >= C) return;
    const uint32_t j = blockIdx.y, b = blockIdx.z, R = gridDim.y;
    const uint32_t Tp = Tn / pt, Hp = Hn / ph, Wp = Wn / pw;
    const uint32_t np = rms_index32(j, order, Tp, Hp, Wp);
    const uint32_t tq = np / (Hp * Wp), hq = (np / Wp) % Hp, wq = np % Wp;
    const size_t N = (size_t)Tn * Hn * Wn;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int dt_ = 0; dt_ < pt; ++dt_)
        for (int dh = 0; dh < ph; ++dh) {
            const size_t row0 = ((size_t)(tq * pt + dt_) * Hn + hq * ph + dh) * Wn + wq * pw;
#pragma unroll 8
            for (int dw = 0; dw < pw; ++dw) {
                const u32x4 v = *(const u32x4 *)(src + ((size_t)b * N + row0 + dw) * C + ch);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += __uint_as_float(v[e] << 16);
                    acc[2 * e + 1] += __uint_as_float(v[e] & 0xffff0000u);
                }
            }
        }
    const float inv = 1.f / (float)(pt * ph * pw);
    O *o = out + ((size_t)b * R + j) * C + ch;
#pragma unroll
    for (int e = 0; e < 8; ++e) elem<O>::store(o + e, acc[e] * inv);
}

} // namespace ssd
} // namespace mate
