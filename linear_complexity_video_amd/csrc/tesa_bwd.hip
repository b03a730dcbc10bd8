// TESA backward on bf16 MFMA (gfx950): the gradients of softmax attention inside
// each (shifted) 3D window. With S = scale Q K^T, P = softmax(S) by rows, O = P V
// and the upstream gradient dO, per window:
//   dV = P^T dO,  dP = dO V^T,  dS_qk = P_qk (dP_qk - delta_q),  delta_q = sum_k P_qk dP_qk,
//   dQ = scale dS K,  dK = scale dS^T Q.
// delta is formed from the kernel's own P and dP rather than as dO . O from the forward's
// bf16 output: where the softmax is peaked, dP - delta cancels and the forward output's
// error shows in dS (dK 1.9% of its rms against 0.4%, unscaled 64-dim inputs).
// dS and P enter the dQ, dK and dV products as pairs of bf16 values (the bf16 rounding and
// the bf16 rounding of what that leaves), two MFMAs on the same operand: these products
// are cancelling sums (the rows of dS sum to zero; dV sums dO rows of mixed sign), and one
// bf16 rounding gave errors of 1.7-2.1% of the gradients' rms (0.4% with the pairs).
// Two kernel templates (three launches), one workgroup per (window, head, block of rows):
//  - k_tesa_bwd_dq: 8 waves, each 32 queries, one per lane column as in the forward
//    (S^T = K Q^T). A first pass over the key tiles gives each query's log-sum-exp and
//    delta (online, against a running maximum); the second forms P^T, dP^T = V dO^T and
//    dS^T, and accumulates dQ^T += K^T dS^T. It also stores (log-sum-exp, delta) per
//    query for the dK and dV kernels.
//  - k_tesa_bwd_dkdv<DK>: 8 waves, each 32 keys, one per lane column (S = Q K^T): per
//    query tile it forms P and accumulates dV^T += dO^T P (DK false), or forms P,
//    dP = dO V^T and dS and accumulates dK^T += Q^T dS (DK true), the transposed
//    tiles read with the LDS transpose read. dV and dK are two launches: together
//    (K, V and both accumulator sets) they need more than the 256 registers of two
//    waves per SIMD, and one wave per SIMD ran slower than recomputing the scores.
// Key or query tiles of 64 rows pass through LDS, the next tile's rows loading
// into registers while the current one is used.
#include "common.hpp"
#include "launch.hpp"
#include "tesa_common.hpp"
#include "timing.hpp"

namespace mate {
namespace {

constexpr int BT = 64;        // rows (keys or queries) per LDS tile
constexpr int NTQ = 512;      // threads of the dQ kernel (8 waves x 32 queries)
constexpr int NTK = 512;      // threads of the dK and dV kernels (8 waves x 32 keys)
constexpr int BPAD = 8;       // tile row padding (bf16)
constexpr int BMAXW = 4096;   // largest window

// Decoded (batch, head, region) of a workgroup and its window.
struct Win {
    int m, t0, h0, w0, nh, nw;
    size_t head_off;
};

__device__ __forceinline__ Win decode_win(int r, int b, int h, int nheads, int DH, int Tn, int Hn, int Wn, int wt,
                                          int wh, int ww, int st, int sh, int sw, int nrh, int nrw)
{
    const int rw = r % nrw, rh = (r / nrw) % nrh, rt = r / (nrw * nrh);
    int t0, t1, h0, h1, w0, w1;
    region_extent(rt, Tn, wt, st, t0, t1);
    region_extent(rh, Hn, wh, sh, h0, h1);
    region_extent(rw, Wn, ww, sw, w0, w1);
    Win X;
    X.nh = h1 - h0;
    X.nw = w1 - w0;
    X.m = (t1 - t0) * X.nh * X.nw;
    X.t0 = t0;
    X.h0 = h0;
    X.w0 = w0;
    X.head_off = ((size_t)b * Tn * Hn * Wn) * ((size_t)nheads * DH) + (size_t)h * DH;
    return X;
}

template <int NT>
__device__ __forceinline__ void build_rows(uint32_t *row, const Win &X, int Hn, int Wn)
{
    const int nhw = X.nh * X.nw;
    const float inv_hw = 1.f / (float)nhw, inv_w = 1.f / (float)X.nw;
    for (int l = threadIdx.x; l < X.m; l += NT) {
        const int lt = div_small(l, nhw, inv_hw);
        const int rem = l - lt * nhw;
        const int lh = div_small(rem, X.nw, inv_w);
        const int lw = rem - lh * X.nw;
        row[l] = (uint32_t)(((X.t0 + lt) * Hn + (X.h0 + lh)) * Wn + (X.w0 + lw));
    }
}

// Row fragment of one token (B operand with the token as column): d = 16 kb + 8 half + 0..7.
template <int DH>
__device__ __forceinline__ void row_frags(const __bf16 *rowp, bf16x8 (&f)[DH / 16])
{
    const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int kb = 0; kb < DH / 16; ++kb) f[kb] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(rowp + 16 * kb + 8 * half));
}

// Tile of BT rows of two tensors through registers: 16-byte chunks, natural layout.
template <int DH, int NT>
struct TilePair {
    static constexpr int DC = DH / 8, PER = BT * DC / NT;
    static_assert(BT * DC % NT == 0, "tile chunks must split evenly over the workgroup");
    u32x4 a[PER], b[PER];
    __device__ __forceinline__ void fetch(const __bf16 *pa, const __bf16 *pb, const uint32_t *row, const Win &X,
                                          int base, size_t rowstride)
    {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int c = threadIdx.x + NT * it, jj = c / DC, dc = c % DC, idx = base + jj;
            // a row past the window reads the window's first row: finite, and masked where used
            const size_t off = X.head_off + (size_t)row[idx < X.m ? idx : 0] * rowstride + 8 * dc;
            a[it] = *(const u32x4 *)(pa + off);
            b[it] = *(const u32x4 *)(pb + off);
        }
    }
    __device__ __forceinline__ void stash(__bf16 (*ta)[DH + BPAD], __bf16 (*tb)[DH + BPAD]) const
    {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int c = threadIdx.x + NT * it;
            *(u32x4 *)&ta[c / DC][8 * (c % DC)] = a[it];
            *(u32x4 *)&tb[c / DC][8 * (c % DC)] = b[it];
        }
    }
};

// Writes one lane's column of a transposed accumulator set (rows: head dims) as a token row.
template <int DH>
__device__ __forceinline__ void store_col(__bf16 *dst, const f32x16 (&acc)[DH / 32], float mul)
{
    const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x4 v4;
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] = (__bf16)(acc[dt][4 * i + j] * mul);
            *(bf16x4 *)(dst + 32 * dt + 8 * i + 4 * half) = v4;
        }
}

template <int DH>
__global__ __launch_bounds__(NTQ) void k_tesa_bwd_dq(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                                                     const __bf16 *__restrict__ v,
                                                     const __bf16 *__restrict__ dout, __bf16 *__restrict__ dq,
                                                     float2 *__restrict__ stats, int nheads, int Tn, int Hn,
                                                     int Wn, int wt, int wh, int ww, int st, int sh, int sw,
                                                     int nrh, int nrw, int nrb, float scale, float c_log2)
{
    __shared__ uint32_t row[BMAXW];
    __shared__ __attribute__((aligned(16))) __bf16 ks[BT][DH + BPAD];
    __shared__ __attribute__((aligned(16))) __bf16 vs[BT][DH + BPAD];

    const int rb = blockIdx.x % nrb, r = blockIdx.x / nrb, h = blockIdx.y, b = blockIdx.z;
    const Win X = decode_win(r, b, h, nheads, DH, Tn, Hn, Wn, wt, wh, ww, st, sh, sw, nrh, nrw);
    const int q_base = rb * NTQ / 2;
    if (q_base >= X.m) return;  // uniform over the workgroup
    build_rows<NTQ>(row, X, Hn, Wn);
    __syncthreads();

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const size_t rowstride = (size_t)nheads * DH;
    const int qi = q_base + wave * 32 + col;
    const bool qvalid = qi < X.m;
    const size_t qoff = X.head_off + (size_t)row[qvalid ? qi : 0] * rowstride;
    bf16x8 qf[DH / 16], dof[DH / 16];
    row_frags<DH>(q + qoff, qf);
    row_frags<DH>(dout + qoff, dof);

    const int ntile = (X.m + BT - 1) / BT;
    // dP^T = V dO^T of the tile in LDS
    auto dprobs = [&](f32x16 (&dp)[2]) {
        dp[0] = f32x16{};
        dp[1] = f32x16{};
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int kb = 0; kb < DH / 16; ++kb)
                dp[sub] = mfma(*(const bf16x8 *)&vs[32 * sub + col][16 * kb + 8 * half], dof[kb], dp[sub]);
    };
    auto scores = [&](int kt, f32x16 (&s)[2]) {
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int kb = 0; kb < DH / 16; ++kb)
                s[sub] = mfma(*(const bf16x8 *)&ks[32 * sub + col][16 * kb + 8 * half], qf[kb], s[sub]);
        // keys past the window get -inf
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int j = kt * BT + 32 * sub + 8 * (rr >> 2) + 4 * half + (rr & 3);
                s[sub][rr] = j < X.m ? s[sub][rr] * c_log2 : -INFINITY;
            }
    };

    // Pass 1: log-sum-exp of each query's scores (log2 units) and delta = sum_k P dP, both
    // against a running maximum; this lane holds half of each tile's keys.
    TilePair<DH, NTQ> tp;
    float mrun = -INFINITY, lrun = 0.f, drun = 0.f;
    tp.fetch(k, v, row, X, 0, rowstride);
    for (int kt = 0; kt < ntile; ++kt) {
        __syncthreads();
        tp.stash(ks, vs);
        __syncthreads();
        tp.fetch(k, v, row, X, (kt + 1 < ntile ? kt + 1 : 0) * BT, rowstride);  // the next tile (pass 2's first)
        f32x16 s[2], dp[2];
        scores(kt, s);
        dprobs(dp);
        float mt = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) mt = fmaxf(mt, s[sub][rr]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mnew = fmaxf(mrun, mt);  // finite: tile 0 holds key 0
        float ls = 0.f, lds = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const float e = __builtin_amdgcn_exp2f(s[sub][rr] - mnew);
                ls += e;
                lds = fmaf(e, dp[sub][rr], lds);
            }
        const float corr = __builtin_amdgcn_exp2f(mrun - mnew);
        lrun = lrun * corr + ls;
        drun = drun * corr + lds;
        mrun = mnew;
    }
    // lanes l and l + 32 hold the two halves of each query's keys
    const float ltot = lrun + __shfl_xor(lrun, 32);
    const float lse = mrun + __log2f(ltot);
    const float delta = (drun + __shfl_xor(drun, 32)) / ltot;

    // Pass 2: dQ^T += K^T dS^T, with P^T = 2^(s - lse) and dS^T = P^T (dP^T - delta).
    f32x16 acc[DH / 32];
#pragma unroll
    for (int i = 0; i < DH / 32; ++i) acc[i] = f32x16{};
    for (int kt = 0; kt < ntile; ++kt) {
        __syncthreads();
        tp.stash(ks, vs);
        __syncthreads();
        if (kt + 1 < ntile) tp.fetch(k, v, row, X, (kt + 1) * BT, rowstride);
        f32x16 s[2], dp[2];
        scores(kt, s);
        dprobs(dp);
        bf16x8 dsh[4], dsl[4];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int rr = 8 * hb + jj;
                    const float p = __builtin_amdgcn_exp2f(s[sub][rr] - lse);
                    const float dsv = p * (dp[sub][rr] - delta);
                    const __bf16 hi = (__bf16)dsv;
                    dsh[2 * sub + hb][jj] = hi;
                    dsl[2 * sub + hb][jj] = (__bf16)(dsv - (float)hi);
                }
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2) {
                const bf16x8 kt_ = v_frag<DH + BPAD>(&ks[0][0], 16 * kb2, 32 * dt);
                acc[dt] = mfma(kt_, dsh[kb2], acc[dt]);
                acc[dt] = mfma(kt_, dsl[kb2], acc[dt]);
            }
    }
    if (qvalid) {
        store_col<DH>(dq + qoff, acc, scale);
        if (half == 0) stats[qoff / DH] = make_float2(lse, delta);
    }
}

template <int DH, bool DK>
__global__ __launch_bounds__(NTK) void k_tesa_bwd_dkdv(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                                                       const __bf16 *__restrict__ v, const __bf16 *__restrict__ dout,
                                                       const float2 *__restrict__ stats, __bf16 *__restrict__ dout_kv,
                                                       int nheads, int Tn, int Hn, int Wn,
                                                       int wt, int wh, int ww, int st, int sh, int sw, int nrh,
                                                       int nrw, int nrb, float scale, float c_log2)
{
    __shared__ uint32_t row[BMAXW];
    __shared__ __attribute__((aligned(16))) __bf16 qs[BT][DH + BPAD];
    __shared__ __attribute__((aligned(16))) __bf16 dos[BT][DH + BPAD];
    __shared__ __attribute__((aligned(16))) float lse_s[BT], del_s[BT];

    const int rb = blockIdx.x % nrb, r = blockIdx.x / nrb, h = blockIdx.y, b = blockIdx.z;
    const Win X = decode_win(r, b, h, nheads, DH, Tn, Hn, Wn, wt, wh, ww, st, sh, sw, nrh, nrw);
    const int k_base = rb * NTK / 2;
    if (k_base >= X.m) return;  // uniform over the workgroup
    build_rows<NTK>(row, X, Hn, Wn);
    __syncthreads();

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const size_t rowstride = (size_t)nheads * DH;
    const int kj = k_base + wave * 32 + col;
    const bool kvalid = kj < X.m;
    const size_t koff = X.head_off + (size_t)row[kvalid ? kj : 0] * rowstride;
    bf16x8 kf[DH / 16], vf[DK ? DH / 16 : 1];
    row_frags<DH>(k + koff, kf);
    if constexpr (DK) row_frags<DH>(v + koff, vf);

    const int ntile = (X.m + BT - 1) / BT;
    f32x16 acc[DH / 32];
#pragma unroll
    for (int i = 0; i < DH / 32; ++i) acc[i] = f32x16{};
    TilePair<DH, NTK> tp;
    float2 stv = make_float2(0.f, 0.f);
    auto fetch_stats = [&](int base) {
        if (tid < BT) {
            const int idx = base + tid;
            stv = stats[(X.head_off + (size_t)row[idx < X.m ? idx : 0] * rowstride) / DH];
        }
    };
    tp.fetch(q, dout, row, X, 0, rowstride);
    fetch_stats(0);
    for (int qt = 0; qt < ntile; ++qt) {
        __syncthreads();
        tp.stash(qs, dos);
        if (tid < BT) {
            lse_s[tid] = stv.x;
            del_s[tid] = stv.y;
        }
        __syncthreads();
        if (qt + 1 < ntile) {
            tp.fetch(q, dout, row, X, (qt + 1) * BT, rowstride);
            fetch_stats((qt + 1) * BT);
        }
        bf16x8 dsh[4], dsl[4];  // dS (DK) or P (dV) as bf16 pairs
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int kb = 0; kb < DH / 16; ++kb) {
                s = mfma(*(const bf16x8 *)&qs[32 * sub + col][16 * kb + 8 * half], kf[kb], s);
                if constexpr (DK) dp = mfma(*(const bf16x8 *)&dos[32 * sub + col][16 * kb + 8 * half], vf[kb], dp);
            }
            // rows of the accumulators: queries 32 sub + 8 i + 4 half + j of this tile
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ql = 32 * sub + 8 * i + 4 * half;
                const float4 l4 = *(const float4 *)&lse_s[ql], d4 = *(const float4 *)&del_s[ql];
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 4 * i + j;
                    const bool ok = qt * BT + ql + j < X.m;
                    const float p = ok ? __builtin_amdgcn_exp2f(s[rr] * c_log2 - lv[j]) : 0.f;
                    const float val = DK ? p * (dp[rr] - dvv[j]) : p;
                    const __bf16 hi = (__bf16)val;
                    dsh[2 * sub + (rr >> 3)][rr & 7] = hi;
                    dsl[2 * sub + (rr >> 3)][rr & 7] = (__bf16)(val - (float)hi);
                }
            }
        }
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2) {
                // dK^T += Q^T dS, or dV^T += dO^T P
                const bf16x8 at = v_frag<DH + BPAD>(DK ? &qs[0][0] : &dos[0][0], 16 * kb2, 32 * dt);
                acc[dt] = mfma(at, dsh[kb2], acc[dt]);
                acc[dt] = mfma(at, dsl[kb2], acc[dt]);
            }
    }
    if (kvalid) store_col<DH>(dout_kv + koff, acc, DK ? scale : 1.f);
}

template <int DH>
hipError_t launch_bwd(const TesaProblem &p, const TesaGradArgs &a, void *ws, hipStream_t st)
{
    const int maxw = p.wt * p.wh * p.ww;
    const int nreg = p.nrt * p.nrh * p.nrw;
    const int nqb = (maxw + NTQ / 2 - 1) / (NTQ / 2), nkb = (maxw + NTK / 2 - 1) / (NTK / 2);
    const float scale = p.scale > 0.f ? p.scale : 1.f / sqrtf((float)DH);
    const float c_log2 = scale * 1.4426950408889634f;
    float2 *stats = (float2 *)ws;
    timing::Scope ts_(K_TESA_BWD, st);
    k_tesa_bwd_dq<DH><<<dim3((unsigned)(nreg * nqb), (unsigned)p.nheads, (unsigned)p.batch), NTQ, 0, st>>>((const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v,
                                             (const __bf16 *)a.dout, (__bf16 *)a.dq, stats,
                                             p.nheads, (int)p.T, (int)p.H, (int)p.W, p.wt, p.wh, p.ww, p.st, p.sh,
                                             p.sw, p.nrh, p.nrw, nqb, scale, c_log2);
    const dim3 gk((unsigned)(nreg * nkb), (unsigned)p.nheads, (unsigned)p.batch);
    k_tesa_bwd_dkdv<DH, false><<<gk, NTK, 0, st>>>((const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v,
                                                    (const __bf16 *)a.dout, stats, (__bf16 *)a.dv, p.nheads, (int)p.T,
                                                    (int)p.H, (int)p.W, p.wt, p.wh, p.ww, p.st, p.sh, p.sw, p.nrh,
                                                    p.nrw, nkb, scale, c_log2);
    k_tesa_bwd_dkdv<DH, true><<<gk, NTK, 0, st>>>((const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v,
                                                   (const __bf16 *)a.dout, stats, (__bf16 *)a.dk, p.nheads, (int)p.T,
                                                   (int)p.H, (int)p.W, p.wt, p.wh, p.ww, p.st, p.sh, p.sw, p.nrh,
                                                   p.nrw, nkb, scale, c_log2);
    return hipGetLastError();
}

} // namespace

bool tesa_backward_supports(const TesaProblem &p)
{
    const int64_t wsize = (int64_t)p.wt * p.wh * p.ww;
    const int64_t blocks = (int64_t)p.nrt * p.nrh * p.nrw * ((wsize + NTK / 2 - 1) / (NTK / 2));
    return p.dtype == 1 && (p.headdim == 64 || p.headdim == 128) && wsize <= BMAXW && blocks < ((int64_t)1 << 31) &&
           p.nheads < 65536 && p.batch < 65536;
}

size_t tesa_backward_workspace(const TesaProblem &p)
{
    return (size_t)p.batch * p.T * p.H * p.W * p.nheads * sizeof(float) * 2;
}

hipError_t tesa_backward(const TesaProblem &p, const TesaGradArgs &a, void *ws, hipStream_t st)
{
    return p.headdim == 64 ? launch_bwd<64>(p, a, ws, st) : launch_bwd<128>(p, a, ws, st);
}

} // namespace mate
