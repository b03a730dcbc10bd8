// Per-token operations of one MATE layer around the core: B, C and dt from
// their joint projection (dt: bias, then softplus) and the MA branch's gated
// RMS norm. The pages give neither the dt activation nor the norm; both follow
// the Mamba2 block the MA branch is built from (softplus keeps dt positive;
// the output is normalised after gating with silu(z)).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mate {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Splits the joint projection's fp32 rows [B | C | dt] (width 2 bc + nheads): B and C rounded to bf16, dt
// as softplus(raw + bias[h]) in fp32. Threads take columns (VEC: groups of 4, which never straddle two of
// the parts when bc and nheads are multiples of 4) of several rows at a time; blocks stride over the rows.
__device__ __forceinline__ float softplus(float u) { return fmaxf(u, 0.f) + log1pf(__expf(-fabsf(u))); }

template <bool VEC>
__global__ __launch_bounds__(256) void k_split_bcdt(const float *__restrict__ src, bf16_t *__restrict__ b,
                                                    bf16_t *__restrict__ c, float *__restrict__ dt,
                                                    const float *__restrict__ bias, int64_t rows, int bc, int nheads)
{
    const int w = 2 * bc + nheads, ncol = VEC ? w / 4 : w;
    const bool wide = ncol >= 256;
    const int rpp = wide ? 1 : 256 / ncol;  // rows per pass
    const int r_in = wide ? 0 : threadIdx.x / ncol, c0 = wide ? threadIdx.x : threadIdx.x % ncol;
    if (r_in >= rpp) return;
    for (int64_t row = (int64_t)blockIdx.x * rpp + r_in; row < rows; row += (int64_t)gridDim.x * rpp)
        for (int cc = c0; cc < ncol; cc += wide ? 256 : ncol) {
            if constexpr (VEC) {
                const int col = 4 * cc;
                const float4 v = *(const float4 *)(src + row * w + col);
                if (col < 2 * bc) {
                    bf16_t *dst = col < bc ? b + row * bc + col : c + row * bc + col - bc;
                    *(uint2 *)dst = make_uint2((uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                                               (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16));
                } else {
                    const int h = col - 2 * bc;
                    const float4 bi = *(const float4 *)(bias + h);
                    *(float4 *)(dt + row * nheads + h) =
                        make_float4(softplus(v.x + bi.x), softplus(v.y + bi.y), softplus(v.z + bi.z), softplus(v.w + bi.w));
                }
            } else {
                const float v = src[row * w + cc];
                if (cc < bc) b[row * bc + cc] = f32_to_bf16(v);
                else if (cc < 2 * bc) c[row * bc + cc - bc] = f32_to_bf16(v);
                else dt[row * nheads + cc - 2 * bc] = softplus(v + bias[cc - 2 * bc]);
            }
        }
}

// Eight bf16 values of a 16-byte piece as floats.
__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8])
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(v[j] << 16);
        f[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
}

__device__ __forceinline__ float silu(float v) { return v / (1.f + __expf(-v)); }

constexpr int NT_NORM = 128;

// One token row per block: g = y * silu(z) over the row's C channels, then per group of gs channels
// out = g / sqrt(mean(g^2) + eps) * w, written over z (bf16). Two passes over the row (rows wider than
// the one-pass kernel's registers hold): the group sums, then the normalised values. gs is a multiple of
// 8, so no 16-byte piece straddles two groups.
__global__ __launch_bounds__(NT_NORM) void k_gated_norm(const bf16_t *__restrict__ y, bf16_t *__restrict__ z,
                                                        const float *__restrict__ w, int C, int G, float eps)
{
    __shared__ float s_part[NT_NORM / 64];
    __shared__ float s_rs[64];  // reciprocal rms per group (G <= 64)
    const size_t row = blockIdx.x;
    const u32x4 *yr = (const u32x4 *)(y + row * C);
    u32x4 *zr = (u32x4 *)(z + row * C);
    const int npc = C / 8, gpc = npc / G;  // pieces per row and per group
    for (int gi = 0; gi < G; ++gi) {
        float acc = 0.f;
        for (int k = gi * gpc + threadIdx.x; k < (gi + 1) * gpc; k += NT_NORM) {
            float fy[8], fz[8];
            unpack8(yr[k], fy);
            unpack8(zr[k], fz);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float gv = fy[j] * silu(fz[j]);
                acc += gv * gv;
            }
        }
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            float t = 0.f;
            for (int k = 0; k < NT_NORM / 64; ++k) t += s_part[k];
            s_rs[gi] = rsqrtf(t / (float)(gpc * 8) + eps);
        }
        __syncthreads();
    }
    for (int k = threadIdx.x; k < npc; k += NT_NORM) {
        float fy[8], fz[8];
        unpack8(yr[k], fy);
        unpack8(zr[k], fz);
        const float rs = s_rs[k / gpc];
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = fy[2 * j] * silu(fz[2 * j]) * rs * w[8 * k + 2 * j];
            const float b = fy[2 * j + 1] * silu(fz[2 * j + 1]) * rs * w[8 * k + 2 * j + 1];
            o[j] = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
        }
        zr[k] = o;
    }
}

// The same in one pass for rows of at most NP * NT_NORM 16-byte pieces: the row's y and z stay in registers
// between the group sums and the output, so each row is read once.
template <int NP>
__global__ __launch_bounds__(NT_NORM) void k_gated_norm_1pass(const bf16_t *__restrict__ y, bf16_t *__restrict__ z,
                                                              const float *__restrict__ w, int C, int G, float eps)
{
    __shared__ float s_part[NT_NORM / 64];
    __shared__ float s_rs[64];
    const size_t row = blockIdx.x;
    const u32x4 *yr = (const u32x4 *)(y + row * C);
    u32x4 *zr = (u32x4 *)(z + row * C);
    const int npc = C / 8, gpc = npc / G;
    u32x4 vy[NP], vz[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int k = threadIdx.x + NT_NORM * j;
        const int kk = k < npc ? k : 0;  // unconditional loads; pieces past the row are not used
        vy[j] = yr[kk];
        vz[j] = zr[kk];
    }
    float sq[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        float fy[8], fz[8];
        unpack8(vy[j], fy);
        unpack8(vz[j], fz);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float gv = fy[e] * silu(fz[e]);
            acc += gv * gv;
        }
        sq[j] = threadIdx.x + NT_NORM * j < npc ? acc : 0.f;
    }
    for (int gi = 0; gi < G; ++gi) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < NP; ++j) acc += (threadIdx.x + NT_NORM * j) / gpc == gi ? sq[j] : 0.f;
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            float t = 0.f;
            for (int k = 0; k < NT_NORM / 64; ++k) t += s_part[k];
            s_rs[gi] = rsqrtf(t / (float)(gpc * 8) + eps);
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int k = threadIdx.x + NT_NORM * j;
        if (k < npc) {
            float fy[8], fz[8];
            unpack8(vy[j], fy);
            unpack8(vz[j], fz);
            const float rs = s_rs[k / gpc];
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = fy[2 * e] * silu(fz[2 * e]) * rs * w[8 * k + 2 * e];
                const float b = fy[2 * e + 1] * silu(fz[2 * e + 1]) * rs * w[8 * k + 2 * e + 1];
                o[e] = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
            }
            zr[k] = o;
        }
    }
}

} // namespace

hipError_t layer_split_bcdt(const float *bcd, void *b, void *c, float *dt, const float *bias, int64_t tokens, int bc,
                            int nheads, hipStream_t st)
{
    if (tokens == 0) return hipSuccess;
    const bool vec = bc % 4 == 0 && nheads % 4 == 0 && ((uintptr_t)bias & 15) == 0;
    const int w = 2 * bc + nheads, ncol = vec ? w / 4 : w;
    const int64_t rpp = ncol >= 256 ? 1 : 256 / ncol;
    const int64_t blocks = std::min<int64_t>((tokens + rpp - 1) / rpp, 8192);
    if (vec)
        k_split_bcdt<true><<<(unsigned)blocks, 256, 0, st>>>(bcd, (bf16_t *)b, (bf16_t *)c, dt, bias, tokens, bc, nheads);
    else
        k_split_bcdt<false><<<(unsigned)blocks, 256, 0, st>>>(bcd, (bf16_t *)b, (bf16_t *)c, dt, bias, tokens, bc, nheads);
    return hipGetLastError();
}

hipError_t layer_gated_norm(const void *y, void *z, const float *w, int64_t tokens, int channels, int groups,
                            float eps, hipStream_t st)
{
    if (tokens == 0) return hipSuccess;
    const int np = (channels / 8 + NT_NORM - 1) / NT_NORM;
    // A block per row, in launches of at most 2^20 rows (a grid of all rows could pass the launch limit
    // of 2^32 work-items).
    constexpr int64_t kRowsPerLaunch = (int64_t)1 << 20;
    for (int64_t r0 = 0; r0 < tokens; r0 += kRowsPerLaunch) {
        const unsigned rows = (unsigned)std::min<int64_t>(kRowsPerLaunch, tokens - r0);
        const bf16_t *yb = (const bf16_t *)y + r0 * channels;
        bf16_t *zb = (bf16_t *)z + r0 * channels;
        if (np <= 2)
            k_gated_norm_1pass<2><<<rows, NT_NORM, 0, st>>>(yb, zb, w, channels, groups, eps);
        else if (np <= 5)
            k_gated_norm_1pass<5><<<rows, NT_NORM, 0, st>>>(yb, zb, w, channels, groups, eps);
        else if (np <= 8)
            k_gated_norm_1pass<8><<<rows, NT_NORM, 0, st>>>(yb, zb, w, channels, groups, eps);
        else
            k_gated_norm<<<rows, NT_NORM, 0, st>>>(yb, zb, w, channels, groups, eps);
    }
    return hipGetLastError();
}

} // namespace mate
