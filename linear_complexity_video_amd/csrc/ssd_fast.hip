// Bidirectional Mamba2 scan on bf16 MFMA (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Same chunked (state space duality) evaluation as the portable path, with
// the chunk states kept on chip. The sequence of each head is cut into
// segments of whole chunks; a workgroup (4 waves) owns one (head, segment):
//
//  1. states   sweeps its segment right to left, carrying the backward state
//              G in MFMA accumulators. Before adding chunk c it stores G (the
//              backward state entering c from the right, from zero at the
//              segment end) as bf16; it also accumulates the segment's forward
//              end state F. Ends with the segment summaries G, F and sum(dt A).
//              The review tokens form one extra segment whose G and F are the
//              initial states of the two directions.
//  2. seg pass turns summaries into the true states at every segment border.
//  3. cb       C_t . B_u (fp32) for every chunk (shared by all heads of a group).
//  4. out      sweeps its segment left to right carrying the forward state Hf
//              and computes, per chunk,
//                 Y^T = X^T M^T + [Hf | Hb] [diag(ef) C | diag(eb) C]^T
//              with M the dense bidirectional intra-chunk matrix (decays below
//              and above the diagonal, 2 C.B dt + 2D on it; fed to the MFMA as
//              an exact hi + lo pair of bf16 fragments), ef = exp(cs),
//              eb = exp(tot - ce), Hb = stored G + decay * border state.
//              Then Hf = exp(tot) Hf + sum_u exp(tot - cs_u) dt_u x_u B_u^T.
// Contractions over tokens need token-contiguous operands, so x and B are
// written to LDS transposed (pairs of tokens per dword); C, CB and the stored
// states are already contiguous along the contraction and are read as MFMA
// fragments straight from memory. Block ids are remapped so that the
// workgroups resident on one XCD work on consecutive heads of one segment and
// share B, C and CB in that XCD's L2.
#include "common.hpp"
#include "launch.hpp"
#include "ssd_common.hpp"

namespace mate {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int P = 64;       // head dim of the MFMA kernels
constexpr int NT = 256;     // threads per workgroup
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// XCD-aware item index of this block (the grid is a multiple of 8).
__device__ __forceinline__ uint32_t xcd_item()
{
    const uint32_t per_xcd = gridDim.x / 8;
    return (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
}

// Loads token pairs (2v, 2v+1) x 16-byte column chunk cc of a chunk of Q rows
// with `cols` bf16 columns per row (x: cols = P per head; B: cols = S per group).
template <int Q, int COLS, bool PERM>
struct PairLoader {
    static constexpr int PAIRS = Q / 2;
    static constexpr int UNITS = PAIRS * (COLS / 8);
    static constexpr int PER = UNITS / NT;
    static_assert(UNITS % NT == 0, "tile must split evenly over the workgroup");
    u32x4 r0[PER], r1[PER];

    // base + row * row_stride + col_off addresses one row's head/group slice.
    __device__ __forceinline__ void load(const __bf16 *base, size_t row_stride, uint32_t c, uint32_t L,
                                         uint32_t batch_rows, int order, uint32_t T, uint32_t H, uint32_t W)
    {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int k = threadIdx.x + NT * it;
            const int v = k % PAIRS, cc = k / PAIRS;
            const uint32_t i0 = c * Q + 2 * v, i1 = i0 + 1;
            r0[it] = u32x4{0, 0, 0, 0};
            r1[it] = u32x4{0, 0, 0, 0};
            if (i0 < L)
                r0[it] = *(const u32x4 *)(base + (batch_rows + ssd::seq_row<PERM>(i0, order, T, H, W)) * row_stride + 8 * cc);
            if (i1 < L)
                r1[it] = *(const u32x4 *)(base + (batch_rows + ssd::seq_row<PERM>(i1, order, T, H, W)) * row_stride + 8 * cc);
        }
    }
    // dst[col][2v..2v+1] (row stride LD bf16) = the pair, optionally scaled by w0 / w1.
    template <int LD>
    __device__ __forceinline__ void store_t(__bf16 *dst, int it) const
    {
        const int k = threadIdx.x + NT * it;
        const int v = k % PAIRS, cc = k / PAIRS;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a0 = r0[it][e], a1 = r1[it][e];
            *(uint32_t *)(dst + (8 * cc + 2 * e) * LD + 2 * v) = (a0 & 0xffffu) | (a1 << 16);
            *(uint32_t *)(dst + (8 * cc + 2 * e + 1) * LD + 2 * v) = (a0 >> 16) | (a1 & 0xffff0000u);
        }
    }
    template <int LD>
    __device__ __forceinline__ void store_t_scaled(__bf16 *dst, int it, float w0, float w1) const
    {
        const int k = threadIdx.x + NT * it;
        const int v = k % PAIRS, cc = k / PAIRS;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a0 = r0[it][e], a1 = r1[it][e];
            *(uint32_t *)(dst + (8 * cc + 2 * e) * LD + 2 * v) = pack2(lo_f(a0) * w0, lo_f(a1) * w1);
            *(uint32_t *)(dst + (8 * cc + 2 * e + 1) * LD + 2 * v) = pack2(hi_f(a0) * w0, hi_f(a1) * w1);
        }
    }
    __device__ __forceinline__ static int pair_of(int it) { return (threadIdx.x + NT * it) % PAIRS; }
};

// ---------------------------------------------------------------------------
// 1. Right-to-left segment sweep: stored backward chunk states + summaries.
// grid = 8 * ceil(batch * nseg * nheads / 8); item = (b * nseg + seg) * nheads + h.
// ---------------------------------------------------------------------------
template <int S, int Q, bool PERM>
__global__ __launch_bounds__(NT) void k_states(const __bf16 *__restrict__ x, const __bf16 *__restrict__ Bm,
                                               const float *__restrict__ dtT, const float *__restrict__ csT,
                                               const float *__restrict__ A, __bf16 *__restrict__ hb_local,
                                               float *__restrict__ delta, float *__restrict__ segF,
                                               float *__restrict__ segB, float *__restrict__ segA, int nheads,
                                               int G, uint32_t L, uint32_t Lpad, int nch, int segch, int nseg,
                                               int seg_base, int nseg_total, int order, uint32_t T, uint32_t H,
                                               uint32_t W, uint32_t total_items)
{
    constexpr int QS = Q + 8;
    __shared__ __bf16 xtb[P * QS];
    __shared__ __bf16 xtf[P * QS];
    __shared__ __bf16 bt[S * QS];

    const uint32_t item = xcd_item();
    if (item >= total_items) return;
    const int h = item % nheads;
    const uint32_t rest = item / nheads;
    const int seg = rest % nseg, b = rest / nseg;
    const int g = h / (nheads / G);
    const int c_lo = seg * segch, c_hi = min(nch, c_lo + segch);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const bool isF = wave >= 2;            // waves 0-1: backward state G^T; 2-3: forward sum F^T
    constexpr int SBW = S / 64;            // s-blocks per wave
    const int sb0 = (wave & 1) * SBW;
    f32x16 acc[SBW][2];
#pragma unroll
    for (int i = 0; i < SBW; ++i) acc[i][0] = acc[i][1] = f32x16{};

    const float a = A[h];
    const size_t drow = ((size_t)b * nheads + h) * Lpad;
    const size_t bh = (size_t)b * nheads + h;
    PairLoader<Q, P, PERM> xl;
    PairLoader<Q, S, PERM> bl;
    float logD = 0.f;  // sum of dt*A over the chunks right of the current one (natural log of the decay)

    for (int c = c_hi - 1; c >= c_lo; --c) {
        xl.load(x + (size_t)h * P, (size_t)nheads * P, c, L, (size_t)b * L, order, T, H, W);
        bl.load(Bm + (size_t)g * S, (size_t)G * S, c, L, (size_t)b * L, order, T, H, W);
        const float tot = csT[drow + (size_t)c * Q + Q - 1];

        // Backward state entering chunk c from the right.
        if (hb_local && !isF) {
            __bf16 *dst = hb_local + (bh * nch + c) * (size_t)(P * S);
#pragma unroll
            for (int i = 0; i < SBW; ++i)
#pragma unroll
                for (int pb = 0; pb < 2; ++pb)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        bf16x4 v4;
#pragma unroll
                        for (int j = 0; j < 4; ++j) v4[j] = (__bf16)acc[i][pb][4 * g4 + j];
                        *(bf16x4 *)(dst + (32 * pb + col) * S + 32 * (sb0 + i) + 8 * g4 + 4 * half) = v4;
                    }
        }
        if (delta && tid == 0) delta[bh * nch + c] = ex2(logD * LOG2E);

        __syncthreads();  // previous chunk's MFMA reads of LDS are done
#pragma unroll
        for (int it = 0; it < xl.PER; ++it) {
            const int v = xl.pair_of(it);
            const size_t i0 = drow + (size_t)c * Q + 2 * v;
            const float d0 = dtT[i0], d1 = dtT[i0 + 1];
            const float c0 = csT[i0], c1 = csT[i0 + 1];
            // backward weights exp(ce) dt, forward weights exp(tot - cs + logD) dt
            xl.template store_t_scaled<QS>(xtb, it, d0 * ex2((c0 - d0 * a) * LOG2E), d1 * ex2((c1 - d1 * a) * LOG2E));
            xl.template store_t_scaled<QS>(xtf, it, d0 * ex2((tot - c0 + logD) * LOG2E),
                                           d1 * ex2((tot - c1 + logD) * LOG2E));
        }
#pragma unroll
        for (int it = 0; it < bl.PER; ++it) bl.template store_t<QS>(bt, it);
        __syncthreads();

        if (!isF) {
            const float dec = ex2(tot * LOG2E);
#pragma unroll
            for (int i = 0; i < SBW; ++i) {
                acc[i][0] *= dec;
                acc[i][1] *= dec;
            }
        }
        const __bf16 *xs = isF ? xtf : xtb;
#pragma unroll
        for (int kb = 0; kb < Q / 16; ++kb) {
            bf16x8 af[SBW], bfr[2];
#pragma unroll
            for (int i = 0; i < SBW; ++i) af[i] = *(const bf16x8 *)&bt[(32 * (sb0 + i) + col) * QS + 16 * kb + 8 * half];
#pragma unroll
            for (int pb = 0; pb < 2; ++pb) bfr[pb] = *(const bf16x8 *)&xs[(32 * pb + col) * QS + 16 * kb + 8 * half];
#pragma unroll
            for (int i = 0; i < SBW; ++i)
#pragma unroll
                for (int pb = 0; pb < 2; ++pb) acc[i][pb] = mfma(af[i], bfr[pb], acc[i][pb]);
        }
        logD += tot;
    }

    float *dst = (isF ? segF : segB) + (bh * nseg_total + seg_base + seg) * (size_t)(P * S);
#pragma unroll
    for (int i = 0; i < SBW; ++i)
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 v4 = {acc[i][pb][4 * g4], acc[i][pb][4 * g4 + 1], acc[i][pb][4 * g4 + 2], acc[i][pb][4 * g4 + 3]};
                *(f32x4 *)(dst + (32 * pb + col) * S + 32 * (sb0 + i) + 8 * g4 + 4 * half) = v4;
            }
    if (tid == 0) segA[bh * nseg_total + seg_base + seg] = logD;
}

// ---------------------------------------------------------------------------
// 2. States at segment borders. grid (ceil(P*S / 256), nheads, batch).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_seg_pass(const float *__restrict__ segF, const float *__restrict__ segB,
                                                  const float *__restrict__ segA, float *__restrict__ hinF,
                                                  float *__restrict__ hinB, int PS, int nseg, int nseg_total,
                                                  int has_review)
{
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= PS) return;
    const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
    const float *F = segF + bh * nseg_total * PS + e;
    const float *Bk = segB + bh * nseg_total * PS + e;
    const float *sa = segA + bh * nseg_total;
    float run = has_review ? F[(size_t)nseg * PS] : 0.f;
    for (int j = 0; j < nseg; ++j) {
        hinF[(bh * nseg + j) * PS + e] = run;
        run = ex2(sa[j] * LOG2E) * run + F[(size_t)j * PS];
    }
    run = has_review ? Bk[(size_t)nseg * PS] : 0.f;
    for (int j = nseg - 1; j >= 0; --j) {
        hinB[(bh * nseg + j) * PS + e] = run;
        run = ex2(sa[j] * LOG2E) * run + Bk[(size_t)j * PS];
    }
}

// ---------------------------------------------------------------------------
// 3. CB[t][u] = C_t . B_u per chunk and group (fp32). grid (nch, G, batch).
// Computed as CB^T = B C^T so each lane holds 4 consecutive u of one t.
// ---------------------------------------------------------------------------
template <int S, int Q>
__global__ __launch_bounds__(NT) void k_cb(const __bf16 *__restrict__ Bm, const __bf16 *__restrict__ Cm,
                                           float *__restrict__ cb, int G, uint32_t L, int order, uint32_t T,
                                           uint32_t H, uint32_t W)
{
    const uint32_t c = blockIdx.x;
    const int g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
    constexpr int TB = Q / 32;
    constexpr int TILES = TB * TB / 4;  // per wave
    const size_t rs = (size_t)G * S;
    float *out = cb + (((size_t)b * G + g) * gridDim.x + c) * (size_t)(Q * Q);
#pragma unroll
    for (int k = 0; k < TILES; ++k) {
        const int ti = wave + 4 * k;
        const int ub = ti / TB, tb = ti % TB;
        const uint32_t iu = c * Q + 32 * ub + col, itk = c * Q + 32 * tb + col;
        const __bf16 *brow = iu < L ? Bm + ((size_t)b * L + rms_index32(iu, order, T, H, W)) * rs + (size_t)g * S : nullptr;
        const __bf16 *crow = itk < L ? Cm + ((size_t)b * L + rms_index32(itk, order, T, H, W)) * rs + (size_t)g * S : nullptr;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kb = 0; kb < S / 16; ++kb) {
            const u32x4 av = brow ? *(const u32x4 *)(brow + 16 * kb + 8 * half) : u32x4{0, 0, 0, 0};
            const u32x4 bv = crow ? *(const u32x4 *)(crow + 16 * kb + 8 * half) : u32x4{0, 0, 0, 0};
            acc = mfma(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc);
        }
        // acc: rows u = 32ub + 8g4 + 4half + j, column t = 32tb + col
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 v4 = {acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2], acc[4 * g4 + 3]};
            *(f32x4 *)(out + (size_t)(32 * tb + col) * Q + 32 * ub + 8 * g4 + 4 * half) = v4;
        }
    }
}

// ---------------------------------------------------------------------------
// 4. Left-to-right output sweep. Same grid/items as k_states (main segments).
// ---------------------------------------------------------------------------
template <int S, int Q>
__global__ __launch_bounds__(NT) void k_out(const __bf16 *__restrict__ x, const __bf16 *__restrict__ Bm,
                                            const __bf16 *__restrict__ Cm, const float *__restrict__ cb,
                                            const float *__restrict__ dtT, const float *__restrict__ csT,
                                            const float *__restrict__ A, const float *__restrict__ Dv,
                                            const __bf16 *__restrict__ hb_local, const float *__restrict__ delta,
                                            const float *__restrict__ hinF, const float *__restrict__ hinB,
                                            __bf16 *__restrict__ y, int nheads, int G, uint32_t N, uint32_t Lpad,
                                            int nch, int segch, int nseg, int order, uint32_t T, uint32_t H,
                                            uint32_t W, uint32_t total_items)
{
    constexpr int QS = Q + 8, SS = S + 8;
    __shared__ __bf16 xt[P * QS];    // x^T
    __shared__ __bf16 xtf[P * QS];   // x^T weighted by dt exp(tot - cs)
    __shared__ __bf16 bt[S * QS];    // B^T
    __shared__ __bf16 hfl[P * SS];   // forward state entering the chunk
    __shared__ __bf16 hbl[P * SS];   // backward state entering the chunk from the right
    __shared__ float s_cs[Q], s_ce[Q], s_dt[Q];  // cs, ce in log2 units

    const uint32_t item = xcd_item();
    if (item >= total_items) return;
    const int h = item % nheads;
    const uint32_t rest = item / nheads;
    const int seg = rest % nseg, b = rest / nseg;
    const int g = h / (nheads / G);
    const int c_lo = seg * segch, c_hi = min(nch, c_lo + segch);
    const size_t bh = (size_t)b * nheads + h;
    const size_t drow = bh * Lpad;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
    // Y^T tiles: Q = 128 -> t-block = wave, p-blocks 0 and 1; Q = 64 -> t-block wave / 2, p-block wave % 2.
    constexpr int YT = Q / 64;
    const int tb = Q == 128 ? wave : wave >> 1;
    const int pb0 = Q == 128 ? 0 : (wave & 1);
    // Hf^T tiles: S = 128 -> s-block = wave, p-blocks 0 and 1; S = 64 -> s-block wave / 2, p-block wave % 2.
    constexpr int HT = S / 64;
    const int hsb = S == 128 ? wave : wave >> 1;
    const int hpb0 = S == 128 ? 0 : (wave & 1);

    const float a = A[h];
    const float twoD = 2.f * Dv[h];
    constexpr int PS = P * S;

    f32x16 hacc[HT];
    {
        const float *src = hinF + (bh * nseg + seg) * (size_t)PS;
#pragma unroll
        for (int i = 0; i < HT; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 v4 = *(const f32x4 *)(src + (32 * (hpb0 + i) + col) * S + 32 * hsb + 8 * g4 + 4 * half);
#pragma unroll
                for (int j = 0; j < 4; ++j) hacc[i][4 * g4 + j] = v4[j];
            }
    }
    // Border state of the backward direction, for this thread's staging chunks.
    constexpr int HBC = PS / 8 / NT;  // 16-byte chunks of Hb per thread
    float hinb[HBC][8];
    {
        const float *src = hinB + (bh * nseg + seg) * (size_t)PS;
#pragma unroll
        for (int it = 0; it < HBC; ++it) {
            const int k = tid + NT * it;
            const f32x4 v0 = *(const f32x4 *)(src + 8 * k), v1 = *(const f32x4 *)(src + 8 * k + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hinb[it][j] = v0[j];
                hinb[it][4 + j] = v1[j];
            }
        }
    }

    PairLoader<Q, P, true> xl;
    PairLoader<Q, S, true> bl;
    const size_t cb_base = ((size_t)b * G + g) * nch;
    const int t_tok = 32 * tb + col;  // this lane's token inside the chunk (Y^T column)

    for (int c = c_lo; c < c_hi; ++c) {
        // ---- global loads ----
        xl.load(x + (size_t)h * P, (size_t)nheads * P, c, N, (size_t)b * N, order, T, H, W);
        bl.load(Bm + (size_t)g * S, (size_t)G * S, c, N, (size_t)b * N, order, T, H, W);
        u32x4 hbr[HBC];
        {
            const __bf16 *src = hb_local + (bh * nch + c) * (size_t)PS;
#pragma unroll
            for (int it = 0; it < HBC; ++it) hbr[it] = *(const u32x4 *)(src + 8 * (tid + NT * it));
        }
        const uint32_t ti = c * Q + t_tok;
        const bool tvalid = ti < N;
        const size_t trow = tvalid ? (size_t)b * N + rms_index32(ti, order, T, H, W) : 0;
        u32x4 cfr[S / 16];
        {
            const __bf16 *crow = Cm + trow * ((size_t)G * S) + (size_t)g * S;
#pragma unroll
            for (int kb = 0; kb < S / 16; ++kb)
                cfr[kb] = tvalid ? *(const u32x4 *)(crow + 16 * kb + 8 * half) : u32x4{0, 0, 0, 0};
        }
        const float *cbrow = cb + (cb_base + c) * (size_t)(Q * Q) + (size_t)t_tok * Q;
        const float tot = csT[drow + (size_t)c * Q + Q - 1];
        const float dl = delta[bh * nch + c];

        __syncthreads();  // previous chunk's LDS reads are done
        // ---- LDS writes ----
#pragma unroll
        for (int it = 0; it < xl.PER; ++it) {
            const int v = xl.pair_of(it);
            const size_t i0 = drow + (size_t)c * Q + 2 * v;
            const float d0 = dtT[i0], d1 = dtT[i0 + 1];
            const float c0 = csT[i0], c1 = csT[i0 + 1];
            xl.template store_t<QS>(xt, it);
            xl.template store_t_scaled<QS>(xtf, it, d0 * ex2((tot - c0) * LOG2E), d1 * ex2((tot - c1) * LOG2E));
        }
#pragma unroll
        for (int it = 0; it < bl.PER; ++it) bl.template store_t<QS>(bt, it);
#pragma unroll
        for (int i = 0; i < HT; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 v4;
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[j] = (__bf16)hacc[i][4 * g4 + j];
                *(bf16x4 *)&hfl[(32 * (hpb0 + i) + col) * SS + 32 * hsb + 8 * g4 + 4 * half] = v4;
            }
#pragma unroll
        for (int it = 0; it < HBC; ++it) {
            const int k = tid + NT * it;
            const int p = k / (S / 8), s0 = 8 * (k % (S / 8));
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack2(lo_f(hbr[it][e]) + dl * hinb[it][2 * e], hi_f(hbr[it][e]) + dl * hinb[it][2 * e + 1]);
            *(u32x4 *)&hbl[p * SS + s0] = o;
        }
        if (tid < Q) {
            const float d = dtT[drow + (size_t)c * Q + tid], cs = csT[drow + (size_t)c * Q + tid];
            s_dt[tid] = d;
            s_cs[tid] = cs * LOG2E;
            s_ce[tid] = (cs - d * a) * LOG2E;
        }
        __syncthreads();

        // ---- Y^T = X^T M^T + [Hf | Hb] [ef C | eb C]^T ----
        const float cs_t = s_cs[t_tok], ce_t = s_ce[t_tok], dt_t = s_dt[t_tok];
        f32x16 yacc[YT];
#pragma unroll
        for (int i = 0; i < YT; ++i) yacc[i] = f32x16{};
#pragma unroll
        for (int kb = 0; kb < Q / 16; ++kb) {
            const int u0 = 16 * kb + 8 * half;
            const f32x4 cb0 = *(const f32x4 *)(cbrow + u0), cb1 = *(const f32x4 *)(cbrow + u0 + 4);
            // M as an exact pair of bf16 fragments (hi + lo), so the intra-chunk
            // product carries fp32-level weights.
            bf16x8 mhi, mlo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int u = u0 + j;
                const float cbv = j < 4 ? cb0[j] : cb1[j - 4];
                float m;
                if (u == t_tok)
                    m = 2.f * cbv * dt_t + twoD;
                else
                    m = cbv * s_dt[u] * ex2(u < t_tok ? cs_t - s_cs[u] : s_ce[u] - ce_t);
                mhi[j] = (__bf16)m;
                mlo[j] = (__bf16)(m - (float)mhi[j]);
            }
#pragma unroll
            for (int i = 0; i < YT; ++i) {
                const bf16x8 af = *(const bf16x8 *)&xt[(32 * (pb0 + i) + col) * QS + u0];
                yacc[i] = mfma(af, mhi, yacc[i]);
                yacc[i] = mfma(af, mlo, yacc[i]);
            }
        }
        {
            const float ef = ex2(cs_t), eb = ex2(tot * LOG2E - ce_t);
#pragma unroll
            for (int kb = 0; kb < S / 16; ++kb) {
                const int s0 = 16 * kb + 8 * half;
                u32x4 fe, fb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float l = lo_f(cfr[kb][e]), hgh = hi_f(cfr[kb][e]);
                    fe[e] = pack2(l * ef, hgh * ef);
                    fb[e] = pack2(l * eb, hgh * eb);
                }
#pragma unroll
                for (int i = 0; i < YT; ++i) {
                    const int prow = 32 * (pb0 + i) + col;
                    yacc[i] = mfma(*(const bf16x8 *)&hfl[prow * SS + s0], __builtin_bit_cast(bf16x8, fe), yacc[i]);
                    yacc[i] = mfma(*(const bf16x8 *)&hbl[prow * SS + s0], __builtin_bit_cast(bf16x8, fb), yacc[i]);
                }
            }
        }

        // ---- Hf = exp(tot) Hf + B^T-weighted x (as Hf^T = B^T xtf^T) ----
        {
            const float dec = ex2(tot * LOG2E);
#pragma unroll
            for (int i = 0; i < HT; ++i) hacc[i] *= dec;
#pragma unroll
            for (int kb = 0; kb < Q / 16; ++kb) {
                const bf16x8 af = *(const bf16x8 *)&bt[(32 * hsb + col) * QS + 16 * kb + 8 * half];
#pragma unroll
                for (int i = 0; i < HT; ++i) {
                    const bf16x8 bfr = *(const bf16x8 *)&xtf[(32 * (hpb0 + i) + col) * QS + 16 * kb + 8 * half];
                    hacc[i] = mfma(af, bfr, hacc[i]);
                }
            }
        }

        // ---- store Y (lane: token t_tok, 4 consecutive p per group) ----
        if (tvalid) {
            __bf16 *yrow = y + (trow * nheads + h) * P;
#pragma unroll
            for (int i = 0; i < YT; ++i)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    bf16x4 v4;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v4[j] = (__bf16)yacc[i][4 * g4 + j];
                    *(bf16x4 *)(yrow + 32 * (pb0 + i) + 8 * g4 + 4 * half) = v4;
                }
        }
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Plan {
    int nseg, segch, nsegT;
    size_t dtT, csT, cb, hbl, delta, segF, segB, segA, hinF, hinB, rx, rB, rdt, rdtT, rcsT, total;
};

Plan make_plan(const SsdProblem &p)
{
    Plan pl{};
    const size_t B = p.batch, Hs = p.nheads, S = p.d_state, Q = p.chunk, PS = (size_t)P * S;
    const size_t Lpad = (size_t)p.nch * Q;
    // About five workgroups per CU over the whole launch.
    int want = (int)((1280 + B * Hs - 1) / (B * Hs));
    if (want < 1) want = 1;
    if (want > p.nch) want = p.nch;
    pl.segch = (p.nch + want - 1) / want;
    pl.nseg = (p.nch + pl.segch - 1) / pl.segch;
    pl.nsegT = pl.nseg + (p.R > 0 ? 1 : 0);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    pl.dtT = take(B * Hs * Lpad * 4);
    pl.csT = take(B * Hs * Lpad * 4);
    pl.cb = take(B * p.ngroups * p.nch * Q * Q * 4);
    pl.hbl = take(B * Hs * p.nch * PS * 2);
    pl.delta = take(B * Hs * p.nch * 4);
    pl.segF = take(B * Hs * pl.nsegT * PS * 4);
    pl.segB = take(B * Hs * pl.nsegT * PS * 4);
    pl.segA = take(B * Hs * pl.nsegT * 4);
    pl.hinF = take(B * Hs * pl.nseg * PS * 4);
    pl.hinB = take(B * Hs * pl.nseg * PS * 4);
    if (p.R > 0) {
        const size_t Rpad = (size_t)p.nchR * Q;
        pl.rx = take(B * p.R * Hs * P * 2);
        pl.rB = take(B * p.R * p.ngroups * S * 2);
        pl.rdt = take(B * p.R * Hs * 4);
        pl.rdtT = take(B * Hs * Rpad * 4);
        pl.rcsT = take(B * Hs * Rpad * 4);
    }
    pl.total = off;
    return pl;
}

unsigned grid_of(uint64_t items) { return (unsigned)((items + 7) / 8 * 8); }

template <int S, int Q>
hipError_t run(const SsdProblem &p, const SsdArgs &a, void *ws, hipStream_t st)
{
    const Plan pl = make_plan(p);
    char *w = (char *)ws;
    float *dtT = (float *)(w + pl.dtT), *csT = (float *)(w + pl.csT);
    float *cb = (float *)(w + pl.cb);
    __bf16 *hbl = (__bf16 *)(w + pl.hbl);
    float *delta = (float *)(w + pl.delta), *segF = (float *)(w + pl.segF), *segB = (float *)(w + pl.segB);
    float *segA = (float *)(w + pl.segA), *hinF = (float *)(w + pl.hinF), *hinB = (float *)(w + pl.hinB);
    const int Hs = p.nheads, G = p.ngroups, Bn = (int)p.batch;
    const uint32_t N = (uint32_t)p.N, Lpad = (uint32_t)(p.nch * Q);
    const uint32_t T = (uint32_t)p.T, H = (uint32_t)p.H, W = (uint32_t)p.W;
    const __bf16 *x = (const __bf16 *)a.x, *Bm = (const __bf16 *)a.b, *Cm = (const __bf16 *)a.c;

    if (p.R > 0) {
        bf16_t *rx = (bf16_t *)(w + pl.rx), *rB = (bf16_t *)(w + pl.rB);
        float *rdt = (float *)(w + pl.rdt), *rdtT = (float *)(w + pl.rdtT), *rcsT = (float *)(w + pl.rcsT);
        const uint32_t R = (uint32_t)p.R, Rpad = (uint32_t)(p.nchR * Q);
        const int64_t Cx = (int64_t)Hs * P, Cb = (int64_t)G * S;
        ssd::k_pool<bf16_t, bf16_t><<<dim3((Cx + 255) / 256, R, Bn), 256, 0, st>>>(
            (const bf16_t *)a.x, rx, Cx, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        ssd::k_pool<bf16_t, bf16_t><<<dim3((Cb + 255) / 256, R, Bn), 256, 0, st>>>(
            (const bf16_t *)a.b, rB, Cb, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        ssd::k_pool<float, float><<<dim3((Hs + 255) / 256, R, Bn), 256, 0, st>>>(
            a.dt, rdt, Hs, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        ssd::k_prep_dt<false><<<dim3(p.nchR, (Hs + 63) / 64, Bn), 256, 0, st>>>(rdt, a.a, rdtT, rcsT, Hs, R, Rpad,
                                                                                Q, 0, 1, 1, R);
        const uint64_t items = (uint64_t)Bn * Hs;
        k_states<S, Q, false><<<grid_of(items), NT, 0, st>>>(
            (const __bf16 *)rx, (const __bf16 *)rB, rdtT, rcsT, a.a, nullptr, nullptr, segF, segB, segA, Hs, G, R,
            Rpad, p.nchR, p.nchR, 1, pl.nseg, pl.nsegT, 0, 1, 1, R, (uint32_t)items);
    }
    ssd::k_prep_dt<true><<<dim3(p.nch, (Hs + 63) / 64, Bn), 256, 0, st>>>(a.dt, a.a, dtT, csT, Hs, N, Lpad, Q,
                                                                         p.order, T, H, W);
    k_cb<S, Q><<<dim3(p.nch, G, Bn), NT, 0, st>>>(Bm, Cm, cb, G, N, p.order, T, H, W);
    const uint64_t items = (uint64_t)Bn * pl.nseg * Hs;
    k_states<S, Q, true><<<grid_of(items), NT, 0, st>>>(x, Bm, dtT, csT, a.a, hbl, delta, segF, segB, segA, Hs, G,
                                                        N, Lpad, p.nch, pl.segch, pl.nseg, 0, pl.nsegT, p.order, T,
                                                        H, W, (uint32_t)items);
    k_seg_pass<<<dim3((P * S + 255) / 256, Hs, Bn), 256, 0, st>>>(segF, segB, segA, hinF, hinB, P * S, pl.nseg,
                                                                  pl.nsegT, p.R > 0 ? 1 : 0);
    k_out<S, Q><<<grid_of(items), NT, 0, st>>>(x, Bm, Cm, cb, dtT, csT, a.a, a.d, hbl, delta, hinF, hinB,
                                               (__bf16 *)a.y, Hs, G, N, Lpad, p.nch, pl.segch, pl.nseg, p.order, T,
                                               H, W, (uint32_t)items);
    return hipGetLastError();
}

} // namespace

bool ssd_fast_supports(const SsdProblem &p)
{
    return p.dtype == 1 && p.headdim == P && (p.d_state == 64 || p.d_state == 128) &&
           (p.chunk == 64 || p.chunk == 128);
}

size_t ssd_fast_workspace(const SsdProblem &p) { return make_plan(p).total; }

hipError_t ssd_fast(const SsdProblem &p, const SsdArgs &a, void *ws, hipStream_t st)
{
    if (p.d_state == 128 && p.chunk == 128) return run<128, 128>(p, a, ws, st);
    if (p.d_state == 64 && p.chunk == 64) return run<64, 64>(p, a, ws, st);
    if (p.d_state == 128 && p.chunk == 64) return run<128, 64>(p, a, ws, st);
    return run<64, 128>(p, a, ws, st);
}

hipError_t ssd_fast_prepare() { return hipSuccess; }

} // namespace mate
