// Bidirectional Mamba (selective scan): the MA branch that the ablation of the xllm-io review
// (Table 2, row "Mamba", and the Mamba2 bullet under it) compares with the Mamba2 scan. Every
// channel c keeps d_state states with their own decay rates,
//   h[c][s] <- exp(dt[c] A[c][s]) h[c][s] + dt[c] x[c] B[s],   y[c] = sum_s C[s] h[c][s] + D[c] x[c],
// so there is no matrix form to put on MFMA (Mamba2's one decay per head is what gives it one):
// the scan is sequential per (channel, state) and bound by the exponentials on the vector ALUs.
// Sequences, review tokens, flip and direction sum are those of the Mamba2 scan.
//
// Work layout: 8 lanes per channel, each holding d_state / 8 states in registers; a workgroup of
// 256 lanes takes 32 channels through the whole sequence (review tokens, then the main tokens in
// scan order); the two directions are separate workgroups of one launch. The scan is bound by
// the vector ALUs, and a SIMD needs two waves to keep them busy (one wave alone stalls on its own
// dependences about half the time): at 5120 channels the two directions make 1280 waves, so every
// SIMD holds one or two (4 lanes per channel, one wave per SIMD, measured slower). Tokens come in
// tiles of 128 through LDS, the next tile's loads in flight while the current one is scanned; the
// rows of a tile's tokens are worked out once, into an LDS table that its loads and stores share.
// Inside a tile, tokens go in groups of 8, stage by stage; the 8 lanes of a channel sum their C h
// terms with three DPP steps. The forward direction writes y, the backward one a partial in the
// workspace, and a last kernel adds the two.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "ssd_common.hpp"
#include "timing.hpp"

namespace mate {
namespace {

constexpr int MB_NT = 256;              // threads per workgroup
constexpr int MB_LPC = 8;               // lanes per channel
constexpr int MB_CPB = MB_NT / MB_LPC;  // channels per workgroup
constexpr int MB_TT = 128;              // tokens per tile
constexpr float MB_LOG2E = 1.4426950408889634f;

// The sum over the 8 lanes of a channel (lanes 8k..8k+7, one half of a 16-lane DPP row) takes three
// DPP steps: mirrored halves (row_half_mirror, 0x141), then the two within-quad swaps (quad_perm
// [1,0,3,2] = 0xB1 and [2,3,0,1] = 0x4E); every lane ends with the total.

// Four consecutive elements as floats, and back.
__device__ __forceinline__ void load4(const float *p, float (&v)[4])
{
    const float4 q = *(const float4 *)p;
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void load4(const bf16_t *p, float (&v)[4])
{
    const uint2 q = *(const uint2 *)p;
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
}
__device__ __forceinline__ void store4(float *p, const float (&v)[4]) { *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ void store4(bf16_t *p, const float (&v)[4])
{
    *(uint2 *)p = make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                             (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
}

// Source of position q of a direction's token stream (review tokens first, then the main tokens):
// review index j (is_review), canonical token n, or nothing past the end.
struct Src {
    uint32_t idx;
    bool review, valid;
};
__device__ __forceinline__ Src token_src(uint32_t q, bool bwd, uint32_t R, uint32_t N, int order, uint32_t T,
                                         uint32_t H, uint32_t W)
{
    if (q < R) return {bwd ? R - 1u - q : q, true, true};
    const uint32_t i = q - R;
    if (i >= N) return {0u, false, false};
    return {rms_index32(bwd ? N - 1u - i : i, order, T, H, W), false, true};
}

// VEC: channels and the x, dt and y pointers allow 4-channel vector access (channels % 4 == 0,
// dt 16-byte aligned); otherwise x, dt and y move one element per access.
template <int S, typename E, bool VEC>
__global__ __launch_bounds__(MB_NT) void k_mamba(const E *__restrict__ x, const E *__restrict__ Bm,
                                                 const E *__restrict__ Cm, const float *__restrict__ dt,
                                                 const float *__restrict__ A, const float *__restrict__ Dv,
                                                 const E *__restrict__ rx, const E *__restrict__ rB,
                                                 const float *__restrict__ rdt, E *__restrict__ yf,
                                                 E *__restrict__ yb, E *__restrict__ trash, int nch, uint32_t N,
                                                 uint32_t R, int order, uint32_t T, uint32_t H, uint32_t W)
{
    constexpr int SPL = S / MB_LPC;                       // states per lane
    constexpr int XPT = MB_TT * MB_CPB / MB_NT;           // x / dt elements per thread per tile
    __shared__ float xs[MB_TT][MB_CPB], ds[MB_TT][MB_CPB], ys[MB_TT][MB_CPB];
    __shared__ float bs[MB_TT][S], cs[MB_TT][S];
    // Source of each token of a tile: canonical row, review row | REV, or ~0u past the end. Two
    // tiles' worth: the one being scanned (its outputs) and the next one (its loads).
    __shared__ uint32_t srow[2][MB_TT];
    constexpr uint32_t REV = 0x80000000u;

    const int tid = threadIdx.x, cl = tid / MB_LPC, sub = tid % MB_LPC;
    const int c0 = blockIdx.x * MB_CPB;
    const uint32_t b = blockIdx.y;
    const bool bwd = blockIdx.z != 0;
    E *out = bwd ? yb : yf;
    const int c = c0 + cl;
    const bool cvalid = c < nch;

    float a2[SPL], h[SPL];
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
        a2[k] = cvalid ? A[(size_t)c * S + sub * SPL + k] * MB_LOG2E : 0.f;
        h[k] = 0.f;
    }
    const float dch = cvalid ? Dv[c] : 0.f;

    const uint32_t L = R + N;
    auto row_of = [&](uint32_t q) -> uint32_t {
        const Src s = token_src(q, bwd, R, N, order, T, H, W);
        return !s.valid ? ~0u : (s.review ? (s.idx | REV) : s.idx);
    };

    // Registers of the next tile. x and dt: VEC, group k = it * 256 + tid holds channels 4 (k % 8)
    // .. + 3 of token k / 8; otherwise element k is channel k % 32 of token k / 32. B and C: group k
    // holds states 4 (k % (S / 4)) .. + 3 of token k / (S / 4). Every load is unconditional: a
    // review token reads the pooled rows; a slot past the end or past the last channel reads
    // element 0 and is zeroed.
    constexpr int XG = VEC ? XPT / 4 : XPT;                       // x / dt loads per thread
    constexpr int BG = (MB_TT * S / 4 + MB_NT - 1) / MB_NT;       // B / C loads per thread
    float rxv[XPT], rdv[XPT], rbv[4 * BG], rcv[4 * BG];
    auto load = [&](const uint32_t *rows) {
#pragma unroll
        for (int it = 0; it < XG; ++it) {
            const int k = it * MB_NT + tid;
            const int tt = VEC ? k / (MB_CPB / 4) : k / MB_CPB, cc = VEC ? 4 * (k % (MB_CPB / 4)) : k % MB_CPB;
            const uint32_t r = rows[tt];
            const bool ok = r != ~0u && c0 + cc < nch, rev = (r & REV) != 0;
            const size_t o = ok ? ((size_t)b * (rev ? R : N) + (r & ~REV)) * nch + c0 + cc : 0;
            if constexpr (VEC) {
                float xv[4], dv[4];
                load4((rev ? rx : x) + o, xv);
                load4((rev ? rdt : dt) + o, dv);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rxv[4 * it + e] = ok ? xv[e] : 0.f;
                    rdv[4 * it + e] = ok ? dv[e] : 0.f;
                }
            } else {
                const float xv = elem<E>::load((rev ? rx : x) + o), dv = (rev ? rdt : dt)[o];
                rxv[it] = ok ? xv : 0.f;
                rdv[it] = ok ? dv : 0.f;
            }
        }
#pragma unroll
        for (int it = 0; it < BG; ++it) {
            const int k = it * MB_NT + tid, tt = (k / (S / 4)) % MB_TT, st = 4 * (k % (S / 4));
            const uint32_t r = rows[tt];
            const bool ok = k < MB_TT * S / 4 && r != ~0u, rev = (r & REV) != 0;
            const size_t o = ok ? ((size_t)b * (rev ? R : N) + (r & ~REV)) * S + st : 0;
            float bv[4], cv[4];
            load4((rev ? rB : Bm) + o, bv);
            load4(Cm + (rev ? 0 : o), cv);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rbv[4 * it + e] = ok ? bv[e] : 0.f;
                rcv[4 * it + e] = ok && !rev ? cv[e] : 0.f;  // review outputs are dropped: C = 0
            }
        }
    };

    if (tid < MB_TT) srow[0][tid] = row_of(tid);
    __syncthreads();
    load(srow[0]);
    int cur = 0;
    for (uint32_t q0 = 0; q0 < L; q0 += MB_TT, cur ^= 1) {
        // the previous tile's scan and output store are done
        __syncthreads();
#pragma unroll
        for (int it = 0; it < XG; ++it) {
            const int k = it * MB_NT + tid;
            if constexpr (VEC) {
                const int tt = k / (MB_CPB / 4), cc = 4 * (k % (MB_CPB / 4));
                *(float4 *)&xs[tt][cc] = make_float4(rxv[4 * it], rxv[4 * it + 1], rxv[4 * it + 2], rxv[4 * it + 3]);
                *(float4 *)&ds[tt][cc] = make_float4(rdv[4 * it], rdv[4 * it + 1], rdv[4 * it + 2], rdv[4 * it + 3]);
            } else {
                xs[k / MB_CPB][k % MB_CPB] = rxv[it];
                ds[k / MB_CPB][k % MB_CPB] = rdv[it];
            }
        }
#pragma unroll
        for (int it = 0; it < BG; ++it) {
            const int k = it * MB_NT + tid;
            if (k < MB_TT * S / 4) {
                const int tt = k / (S / 4), st = 4 * (k % (S / 4));
                *(float4 *)&bs[tt][st] = make_float4(rbv[4 * it], rbv[4 * it + 1], rbv[4 * it + 2], rbv[4 * it + 3]);
                *(float4 *)&cs[tt][st] = make_float4(rcv[4 * it], rcv[4 * it + 1], rcv[4 * it + 2], rcv[4 * it + 3]);
            }
        }
        const bool more = q0 + MB_TT < L;
        if (more && tid < MB_TT) srow[cur ^ 1][tid] = row_of(q0 + MB_TT + tid);
        __syncthreads();
        if (more) load(srow[cur ^ 1]);  // in flight during the scan of this tile

        // Groups of GS tokens without a branch: every lane of a channel ends a token with its y, and
        // lane j % 8 keeps that of token j, so the group's results leave in one store per lane.
        constexpr int GS = 8, KPL = GS / MB_LPC;
        // Stage by stage over the group's tokens (decays and inputs, the state chain, the C h
        // products, each DPP step), so that a wave has independent work in flight.
        for (int t0 = 0; t0 < MB_TT; t0 += GS) {
            float gd[GS], gx[GS], e[GS][SPL], u[GS][SPL], acc[GS];
#pragma unroll
            for (int j = 0; j < GS; ++j) {
                gd[j] = ds[t0 + j][cl];
                gx[j] = xs[t0 + j][cl];
                const float dx = gd[j] * gx[j];
#pragma unroll
                for (int k = 0; k < SPL; ++k) {
                    e[j][k] = __builtin_amdgcn_exp2f(gd[j] * a2[k]);
                    u[j][k] = dx * bs[t0 + j][sub * SPL + k];
                }
            }
#pragma unroll
            for (int j = 0; j < GS; ++j) {
                acc[j] = 0.f;
#pragma unroll
                for (int k = 0; k < SPL; ++k) {
                    h[k] = fmaf(e[j][k], h[k], u[j][k]);
                    acc[j] = fmaf(cs[t0 + j][sub * SPL + k], h[k], acc[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < GS; ++j)
                acc[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[j]), 0x141, 0xF, 0xF, false));
#pragma unroll
            for (int j = 0; j < GS; ++j)
                acc[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[j]), 0xB1, 0xF, 0xF, false));
#pragma unroll
            for (int j = 0; j < GS; ++j)
                acc[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[j]), 0x4E, 0xF, 0xF, false));
            float keep[KPL];
#pragma unroll
            for (int m = 0; m < KPL; ++m) keep[m] = 0.f;
#pragma unroll
            for (int j = 0; j < GS; ++j)
                keep[j / MB_LPC] = sub == j % MB_LPC ? fmaf(dch, gx[j], acc[j]) : keep[j / MB_LPC];
#pragma unroll
            for (int m = 0; m < KPL; ++m) ys[t0 + m * MB_LPC + sub][cl] = keep[m];
        }
        __syncthreads();

        // Output of the main tokens of this tile, at their canonical rows.
#pragma unroll
        for (int it = 0; it < XG; ++it) {
            const int k = it * MB_NT + tid;
            const int tt = VEC ? k / (MB_CPB / 4) : k / MB_CPB, cc = VEC ? 4 * (k % (MB_CPB / 4)) : k % MB_CPB;
            const uint32_t r = srow[cur][tt];
            const bool ok = r != ~0u && !(r & REV) && c0 + cc < nch;
            E *dst = ok ? out + ((size_t)b * N + r) * nch + c0 + cc : trash + 4 * (tid & 63);
            if constexpr (VEC) {
                const float4 v = *(const float4 *)&ys[tt][cc];
                const float v4[4] = {v.x, v.y, v.z, v.w};
                store4(dst, v4);
            } else {
                elem<E>::store(dst, ys[tt][cc]);
            }
        }
    }
}

// y = y + partial (the two directions), elementwise over `total` elements; 16 bytes per access
// when `total` is a multiple of the vector width (y and the partial are 16-byte aligned).
template <typename E>
__global__ __launch_bounds__(256) void k_mamba_sum(E *__restrict__ y, const E *__restrict__ part, size_t total)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int V = 16 / sizeof(E);
    const size_t stride = (size_t)gridDim.x * 256;
    if (total % V == 0) {
        for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total / V; i += stride) {
            u32x4 a = ((const u32x4 *)y)[i];
            const u32x4 p = __builtin_nontemporal_load((const u32x4 *)part + i);
            E *ae = (E *)&a;
            const E *pe = (const E *)&p;
#pragma unroll
            for (int e = 0; e < V; ++e) elem<E>::store(ae + e, elem<E>::load(ae + e) + elem<E>::load(pe + e));
            ((u32x4 *)y)[i] = a;
        }
    } else {
        for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride)
            elem<E>::store(y + i, elem<E>::load(y + i) + elem<E>::load(part + i));
    }
}

template <typename E>
hipError_t run(const MambaProblem &p, const MambaArgs &a, void *ws, hipStream_t st)
{
    const uint32_t T = (uint32_t)p.T, H = (uint32_t)p.H, W = (uint32_t)p.W;
    const uint32_t N = (uint32_t)(p.T * p.H * p.W), R = (uint32_t)p.R;
    const int Bn = (int)p.batch, C = p.channels, S = p.d_state;
    char *w = (char *)ws;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char *q = w + off;
        off += (bytes + 255) & ~(size_t)255;
        return q;
    };
    E *part = (E *)take((size_t)Bn * N * C * sizeof(E));
    E *trash = (E *)take(256 * sizeof(E));
    // Pooled review tokens: x and B in the input dtype (so that one load serves review and main
    // tokens), dt in fp32. Without review tokens the pointers only need to be readable.
    const E *rx = (const E *)a.x, *rB = (const E *)a.b;
    const float *rdt = a.dt;
    if (R > 0) {
        E *px = (E *)take((size_t)Bn * R * C * sizeof(E));
        float *pdt = (float *)take((size_t)Bn * R * C * 4);
        E *pB = (E *)take((size_t)Bn * R * S * sizeof(E));
        timing::Scope ts_(K_SSD_POOL, st);
        // bf16 rows of whole 16-byte pieces pool 8 channels per thread
        auto pool_rows = [&](const E *src, E *dst, int64_t Cr) {
            if constexpr (std::is_same<E, bf16_t>::value) {
                if (Cr % 8 == 0 && ((uintptr_t)src & 15) == 0) {
                    ssd::k_pool8<bf16_t><<<dim3((unsigned)((Cr + 2047) / 2048), R, Bn), 256, 0, st>>>(
                        src, dst, Cr, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
                    return;
                }
            }
            ssd::k_pool<E, E><<<dim3((unsigned)((Cr + 255) / 256), R, Bn), 256, 0, st>>>(src, dst, Cr, T, H, W, p.pool_t,
                                                                                       p.pool_h, p.pool_w, p.order);
        };
        pool_rows((const E *)a.x, px, C);
        if (ssd::pool_f32x4_ok(a.dt, C))
            ssd::k_pool_f32x4<<<dim3(R, Bn), ssd::kPoolF4Threads, 0, st>>>(a.dt, pdt, C, T, H, W, p.pool_t, p.pool_h,
                                                                         p.pool_w, p.order);
        else if (C % 4 == 0 && ((uintptr_t)a.dt & 15) == 0)
            ssd::k_pool_f32x4_wide<<<dim3((unsigned)((C + 1023) / 1024), R, Bn), 256, 0, st>>>(
                a.dt, pdt, C, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        else
            ssd::k_pool<float, float><<<dim3((C + 255) / 256, R, Bn), 256, 0, st>>>(a.dt, pdt, C, T, H, W, p.pool_t,
                                                                                   p.pool_h, p.pool_w, p.order);
        pool_rows((const E *)a.b, pB, S);
        rx = px;
        rdt = pdt;
        rB = pB;
    }
    const dim3 grid((C + MB_CPB - 1) / MB_CPB, Bn, 2);
    {
        timing::Scope ts_(K_MAMBA, st);
        // 4-channel access needs every row of x, dt, y (and of the pooled x, dt) 16-byte aligned
        // for dt and 8- or 16-byte aligned for x and y: channels % 4 == 0 and a 16-byte aligned dt.
        const bool vec = C % 4 == 0 && ((uintptr_t)a.dt & 15) == 0;
#define MB_LAUNCH(SS, VV)                                                                                             \
    k_mamba<SS, E, VV><<<grid, MB_NT, 0, st>>>((const E *)a.x, (const E *)a.b, (const E *)a.c, a.dt, a.a, a.d, rx,   \
                                               rB, rdt, (E *)a.y, part, trash, C, N, R, p.order, T, H, W)
        if (vec) {
            switch (S) {
            case 8: MB_LAUNCH(8, true); break;
            case 16: MB_LAUNCH(16, true); break;
            default: MB_LAUNCH(32, true); break;
            }
        } else {
            switch (S) {
            case 8: MB_LAUNCH(8, false); break;
            case 16: MB_LAUNCH(16, false); break;
            default: MB_LAUNCH(32, false); break;
            }
        }
#undef MB_LAUNCH
    }
    const size_t total = (size_t)Bn * N * C;
    const size_t want = (total + 255) / 256;
    const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
    k_mamba_sum<E><<<blocks, 256, 0, st>>>((E *)a.y, part, total);
    return hipGetLastError();
}

} // namespace

size_t mamba_workspace(const MambaProblem &p)
{
    const size_t e = p.dtype == 1 ? 2 : 4;
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t N = (size_t)(p.T * p.H * p.W);
    size_t s = al((size_t)p.batch * N * p.channels * e) + al(256 * e);
    if (p.R > 0)
        s += al((size_t)p.batch * p.R * p.channels * e) + al((size_t)p.batch * p.R * p.channels * 4) +
             al((size_t)p.batch * p.R * p.d_state * e);
    return s;
}

hipError_t mamba_scan(const MambaProblem &p, const MambaArgs &a, void *ws, hipStream_t st)
{
    return p.dtype == 1 ? run<bf16_t>(p, a, ws, st) : run<float>(p, a, ws, st);
}

} // namespace mate
