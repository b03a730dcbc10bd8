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
// dt * A. Positions >= L are zero (exact no-ops of the recurrence). The rows of
// a chunk come from `perm` when given (scan position -> canonical token), else
// from the RMS index (PERM) or the identity.
// grid (nchunks, ceil(nheads / kPrepHeads), batch), kPrepThreads threads; Q <= 128. VEC: the heads of
// a token row are read as 16-byte pieces (nheads a multiple of 4, dt 16-byte aligned).
constexpr int kPrepHeads = 128, kPrepThreads = 512;
template <bool PERM, bool VEC>
__global__ __launch_bounds__(kPrepThreads) void k_prep_dt(const float *__restrict__ dt, const float *__restrict__ A,
                                                          float *__restrict__ dtT, float *__restrict__ csT, int nheads,
                                                          uint32_t L, uint32_t Lpad, int Q, int order, uint32_t T,
                                                          uint32_t H, uint32_t W, const uint32_t *__restrict__ perm)
{
    __shared__ float sdt[kMaxQ][kPrepHeads + 1];
    __shared__ uint32_t srow[kMaxQ];
    const uint32_t c = blockIdx.x, b = blockIdx.z;
    const int h0 = blockIdx.y * kPrepHeads, nh = min(kPrepHeads, nheads - h0);
    const int tid = threadIdx.x;
    // The chunk's rows first, so that the dt loads below depend on no other load and
    // can all be in flight together.
    for (int u = tid; u < Q; u += kPrepThreads) {
        const uint32_t i = c * Q + u;
        srow[u] = i < L ? (perm ? perm[i] : seq_row<PERM>(i, order, T, H, W)) : ~0u;
    }
    __syncthreads();
    // Each thread keeps one column (a 16-byte piece, or one head) and walks the rows.
    const int ncol = VEC ? nh / 4 : nh;
    const int rpp = kPrepThreads / ncol, j = tid % ncol;  // rows per pass (ncol <= kPrepThreads)
    for (int u = tid / ncol; u < Q && tid < rpp * ncol; u += rpp) {
        const uint32_t row = srow[u];
        const float *src = dt + ((size_t)b * L + (row != ~0u ? row : 0u)) * nheads + h0;
        if constexpr (VEC) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row != ~0u) v = *(const float4 *)(src + 4 * j);
            sdt[u][4 * j] = v.x;
            sdt[u][4 * j + 1] = v.y;
            sdt[u][4 * j + 2] = v.z;
            sdt[u][4 * j + 3] = v.w;
        } else {
            sdt[u][j] = row != ~0u ? src[j] : 0.f;
        }
    }
    __syncthreads();
    // One wave per head at a time: lane l owns positions 2l and 2l + 1; a wave-wide
    // inclusive scan of the lane sums gives the cumulative sums.
    const int lane = tid & 63, wave = tid >> 6;
    for (int hh = wave; hh < nh; hh += kPrepThreads / 64) {
        const int h = h0 + hh;
        const float a = A[h];
        const int u0 = 2 * lane;
        const float d0 = u0 < Q ? sdt[u0][hh] : 0.f, d1 = u0 + 1 < Q ? sdt[u0 + 1][hh] : 0.f;
        const float v0 = d0 * a, v1 = d1 * a;
        float run = v0 + v1;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(run, off, 64);
            if (lane >= off) run += o;
        }
        const float cs1 = run, cs0 = run - v1;
        if (u0 < Q) {
            const size_t o = ((size_t)b * nheads + h) * Lpad + (size_t)c * Q + u0;
            if (u0 + 1 < Q && (Q & 1) == 0) {  // o is even: 8-byte aligned pair
                *(float2 *)(dtT + o) = make_float2(d0, d1);
                *(float2 *)(csT + o) = make_float2(cs0, cs1);
            } else {
                dtT[o] = d0;
                csT[o] = cs0;
                if (u0 + 1 < Q) {
                    dtT[o + 1] = d1;
                    csT[o + 1] = cs1;
                }
            }
        }
    }
}

// Launches k_prep_dt for nch chunks of Q positions.
template <bool PERM>
inline void prep_dt(const float *dt, const float *A, float *dtT, float *csT, int nheads, uint32_t L, uint32_t Lpad,
                    int Q, int order, uint32_t T, uint32_t H, uint32_t W, uint32_t nch, uint32_t batch,
                    hipStream_t st, const uint32_t *perm = nullptr)
{
    const dim3 grid(nch, (unsigned)((nheads + kPrepHeads - 1) / kPrepHeads), batch);
    if (nheads % 4 == 0 && ((uintptr_t)dt & 15) == 0)
        k_prep_dt<PERM, true><<<grid, kPrepThreads, 0, st>>>(dt, A, dtT, csT, nheads, L, Lpad, Q, order, T, H, W, perm);
    else
        k_prep_dt<PERM, false><<<grid, kPrepThreads, 0, st>>>(dt, A, dtT, csT, nheads, L, Lpad, Q, order, T, H, W, perm);
}

// Whether k_pool_f32x4 applies: 16-byte aligned rows of at most 1024 channels.
inline bool pool_f32x4_ok(const float *src, int C)
{
    return C % 4 == 0 && C / 4 <= 256 && ((uintptr_t)src & 15) == 0;
}

// Average pool of fp32 rows, 4 channels per thread, many pooled tokens' rows
// read in parallel per block and reduced through LDS in two rounds. C must be a
// multiple of 4 and C / 4 <= 256. out[b][j][ch] with j in RMS order `order` of
// the pooled grid. grid (R, batch), kPoolF4Threads threads.
constexpr int kPoolF4Threads = 1024;
template <typename F = float>
__global__ __launch_bounds__(kPoolF4Threads) void k_pool_f32x4(const F *__restrict__ src, F *__restrict__ out, int C,
                                                               uint32_t Tn, uint32_t Hn, uint32_t Wn, int pt, int ph,
                                                               int pw, int order)
{
    constexpr int NT = kPoolF4Threads, NP = 8;  // threads; partial sums per channel group after round one
    __shared__ float4 part[NT];
    __shared__ float4 part2[NP * 256];
    const int cg = C / 4, rp = NT / cg;  // channel groups; rows in flight
    const int r = threadIdx.x / cg, g = threadIdx.x % cg;
    const uint32_t j = blockIdx.x, b = blockIdx.y, R = gridDim.x;
    const uint32_t Tp = Tn / pt, Hp = Hn / ph, Wp = Wn / pw;
    const uint32_t np = rms_index32(j, order, Tp, Hp, Wp);
    const uint32_t tq = np / (Hp * Wp), hq = (np / Wp) % Hp, wq = np % Wp;
    const size_t N = (size_t)Tn * Hn * Wn;
    const int cnt = pt * ph * pw;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < rp) {
        for (int e = r; e < cnt; e += rp) {
            const int dw = e % pw, dh = (e / pw) % ph, dt_ = e / (pw * ph);
            const size_t n = ((size_t)(tq * pt + dt_) * Hn + hq * ph + dh) * Wn + wq * pw + dw;
            const float4 v = *(const float4 *)(src + ((size_t)b * N + n) * C + 4 * g);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    // round one: np2 partial sums per channel group, each over every np2-th row slot (np2 cg <= NT)
    const int np2 = min(NP, NT / cg);
    if (threadIdx.x < np2 * cg) {
        const int gg = threadIdx.x % cg, k0 = threadIdx.x / cg;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k = k0; k < rp; k += np2) {
            const float4 v = part[k * cg + gg];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        part2[threadIdx.x] = s;
    }
    __syncthreads();
    if (threadIdx.x < cg) {
        float4 s = part2[threadIdx.x];
        for (int k = 1; k < np2; ++k) {
            const float4 v = part2[k * cg + threadIdx.x];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        const float inv = 1.f / (float)cnt;
        *(float4 *)(out + ((size_t)b * R + j) * C + 4 * threadIdx.x) =
            make_float4(s.x * inv, s.y * inv, s.z * inv, s.w * inv);
    }
}

// Average pool of wide fp32 rows (C a multiple of 4, rows 16-byte aligned): 4 channels per thread, each
// thread walking its pool block's rows in the order of k_pool (so the sums are the same). grid
// (ceil(C / 1024), R, batch).
template <typename F = float>
__global__ __launch_bounds__(256) void k_pool_f32x4_wide(const F *__restrict__ src, F *__restrict__ out,
                                                        int64_t C, uint32_t Tn, uint32_t Hn, uint32_t Wn, int pt,
                                                        int ph, int pw, int order)
{
    const int64_t ch = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (ch >= C) return;
    const uint32_t j = blockIdx.y, b = blockIdx.z, R = gridDim.y;
    const uint32_t Tp = Tn / pt, Hp = Hn / ph, Wp = Wn / pw;
    const uint32_t np = rms_index32(j, order, Tp, Hp, Wp);
    const uint32_t tq = np / (Hp * Wp), hq = (np / Wp) % Hp, wq = np % Wp;
    const size_t N = (size_t)Tn * Hn * Wn;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int dt_ = 0; dt_ < pt; ++dt_)
        for (int dh = 0; dh < ph; ++dh) {
            const size_t row0 = ((size_t)(tq * pt + dt_) * Hn + hq * ph + dh) * Wn + wq * pw;
#pragma unroll 8
            for (int dw = 0; dw < pw; ++dw) {
                typedef float f32x4v __attribute__((ext_vector_type(4)));
                const f32x4v v = __builtin_nontemporal_load((const f32x4v *)(src + ((size_t)b * N + row0 + dw) * C + ch));
                acc.x += v[0]; acc.y += v[1]; acc.z += v[2]; acc.w += v[3];
            }
        }
    const float inv = 1.f / (float)(pt * ph * pw);
    *(float4 *)(out + ((size_t)b * R + j) * C + ch) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
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
// thread; C must be a multiple of 8. Narrow rows (C / 8 < 256) are split over
// several row slots of the block, reduced through LDS. Output bf16 (rounded) or
// fp32. grid (ceil(C / 2048), R, batch).
template <typename O>
__global__ __launch_bounds__(256) void k_pool8(const bf16_t *__restrict__ src, O *__restrict__ out, int64_t C,
                                               uint32_t Tn, uint32_t Hn, uint32_t Wn, int pt, int ph, int pw,
                                               int order)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ float part[256][9];
    const int64_t groups = C / 8;
    const int cg = groups < 256 ? (int)groups : 256;  // channel groups per block
    const int rp = 256 / cg;                          // row slots
    const int r = threadIdx.x / cg, gi = threadIdx.x % cg;
    const int64_t ch = ((int64_t)blockIdx.x * 256 + gi) * 8;
    const uint32_t j = blockIdx.y, b = blockIdx.z, R = gridDim.y;
    const uint32_t Tp = Tn / pt, Hp = Hn / ph, Wp = Wn / pw;
    const uint32_t np = rms_index32(j, order, Tp, Hp, Wp);
    const uint32_t tq = np / (Hp * Wp), hq = (np / Wp) % Hp, wq = np % Wp;
    const size_t N = (size_t)Tn * Hn * Wn;
    const int cnt = pt * ph * pw;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (rp == 1) {  // wide rows: one slot walks the whole pool block
        if (ch < C)
            for (int dt_ = 0; dt_ < pt; ++dt_)
                for (int dh = 0; dh < ph; ++dh) {
                    const size_t row0 = ((size_t)(tq * pt + dt_) * Hn + hq * ph + dh) * Wn + wq * pw;
#pragma unroll 8
                    for (int dw = 0; dw < pw; ++dw) {
                        // read once: streaming loads leave L2 to the kernels running beside
                        const u32x4 v = __builtin_nontemporal_load((const u32x4 *)(src + ((size_t)b * N + row0 + dw) * C + ch));
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2) {
                            acc[2 * e2] += __uint_as_float(v[e2] << 16);
                            acc[2 * e2 + 1] += __uint_as_float(v[e2] & 0xffff0000u);
                        }
                    }
                }
    } else if (r < rp && ch < C) {
#pragma unroll 4
        for (int e = r; e < cnt; e += rp) {
            const int dw = e % pw, dh = (e / pw) % ph, dt_ = e / (pw * ph);
            const size_t n = ((size_t)(tq * pt + dt_) * Hn + hq * ph + dh) * Wn + wq * pw + dw;
            const u32x4 v = __builtin_nontemporal_load((const u32x4 *)(src + ((size_t)b * N + n) * C + ch));
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                acc[2 * e2] += __uint_as_float(v[e2] << 16);
                acc[2 * e2 + 1] += __uint_as_float(v[e2] & 0xffff0000u);
            }
        }
    }
    const float inv = 1.f / (float)cnt;
    if (rp == 1) {
        if (ch < C) {
            O *o = out + ((size_t)b * R + j) * C + ch;
#pragma unroll
            for (int e = 0; e < 8; ++e) elem<O>::store(o + e, acc[e] * inv);
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[threadIdx.x][e] = acc[e];
    __syncthreads();
    if (threadIdx.x < cg && ch < C) {
        O *o = out + ((size_t)b * R + j) * C + ch;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float sum = 0.f;
            for (int k = 0; k < rp; ++k) sum += part[k * cg + threadIdx.x][e];
            elem<O>::store(o + e, sum * inv);
        }
    }
}

} // namespace ssd
} // namespace mate
