// Bidirectional Mamba2 scan on bf16 MFMA (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Same chunked (state space duality) evaluation as the portable path, with
// the chunk states kept on chip. The sequence of each head is cut into
// segments of whole chunks; a workgroup of four waves (two workgroups per CU)
// owns one (head, segment) in the two sweeps:
//
//  1. states   sweeps its segment right to left, carrying the backward state
//              G in MFMA accumulators. Before adding chunk c it stores G (the
//              backward state entering c from the right, from zero at the
//              segment end) as bf16; it also accumulates the segment's forward
//              end state F. Ends with the segment summaries G, F and sum(dt A).
//              The review tokens form one extra segment whose G and F are the
//              initial states of the two directions.
//  2. seg pass turns summaries into the true states at every segment border.
//  3. cb       per chunk and group (shared by its heads): C_t . B_u (fp16), and
//              B^T, C and CB in MFMA operand order (used by 1 and 4).
//  4. out      sweeps its segment left to right carrying the forward state Hf
//              and computes, per chunk,
//                 Y^T = X^T M^T + ef * (Hf C^T) + eb * (Hb C^T)
//              with M the dense bidirectional intra-chunk matrix (decays below
//              and above the diagonal, 2 C.B dt + 2D on it), ef = exp(cs),
//              eb = exp(tot - ce) applied per token to the accumulators, and
//              Hb = stored G + decay * border state. X^T M^T runs on fp16
//              MFMA (x is converted exactly, M rounded to fp16): its weights
//              are the largest values of the scan and fp16 keeps 3 more
//              mantissa bits than bf16.
//              Then Hf = exp(tot) Hf + sum_u exp(tot - cs_u) dt_u x_u B_u^T.
//
// Data layout: operands with one consumer wave (B^T of a state block, C and CB
// of a token block) are stored per chunk in MFMA operand order, 1 KB per
// k-block, and loaded straight into registers (one contiguous load per wave).
// x, whose operands every wave reads, and the two states of the output sweep
// are staged in LDS in row-major layout; x operands of the contractions over
// tokens are read with the gfx950 LDS transpose read (ds_read_b64_tr_b16),
// which hands each lane 4 consecutive rows of one column.
//
// Decay weights of M: each lane builds its M^T operand (its token's row, 8
// consecutive u) in registers from its CB piece. Inside the 32x32 diagonal
// block each weight is one exp2; in the blocks below (above) it, exp(cs_t -
// cs_u) (exp(ce_u - ce_t)) is split at the block edge into a per-lane factor
// and a per-token factor, both <= 1, so no exponent is evaluated per element.
//
// Scan order: a table of the RMS permutation (scan position -> canonical
// token) is built once per call; every gather reads it instead of dividing.
// Block ids are remapped so that the workgroups resident on one XCD work on
// consecutive heads of one segment and share B, C and CB in that XCD's L2.
#include "common.hpp"
#include "launch.hpp"
#include "mfma_frag.hpp"
#include "ssd_common.hpp"
#include "timing.hpp"

namespace mate {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int P = 64;       // head dim of the MFMA kernels
constexpr int NT = 256;     // threads per workgroup
constexpr int XPAD = 32;    // LDS row padding (bf16) of token-row tiles
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma16(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

__device__ __forceinline__ uint32_t pack2h(float a, float b)
{
    f16x2 r;
    r[0] = (_Float16)a;
    r[1] = (_Float16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float h_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of the lane 8 apart in the same row of 16 lanes (a rotation by 8 within the row, i.e. lane ^ 8).
__device__ __forceinline__ float dpp_ror8(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
}

// Pins a value at this point of the program: an empty volatile asm that reads and redefines it, so the
// compiler cannot compute with the value (and wait for the load that produced it) any earlier.
template <typename T>
__device__ __forceinline__ void pin(T &v)
{
    asm volatile("" : "+v"(v));
}

// XCD-aware item index of this block (the grid is a multiple of 8).
__device__ __forceinline__ uint32_t xcd_item()
{
    const uint32_t per_xcd = gridDim.x / 8;
    return (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
}

using frag::frag_rm;
using frag::frag_tr;

// Q token rows of COLS bf16 each, split in 16-byte units over the workgroup.
// Row u of the chunk is read from global row srow[u] (an LDS table of the
// chunk's rows; ~0u marks a position past the end). Loads are unconditional:
// a position past the end reads row 0 of the batch, a finite row that the
// kernels multiply by that position's weight dt = 0 (or never store), so no
// select waits on the load.
// GROUPED: the four pieces of a thread are four rows of one aligned group of 8 rows (rows 8 g + 2 it +
// (r8 & 1), g = 4 wave + r8 / 2, r8 = lane / 8), so that a thread sums its pieces and one exchange with
// the lane 8 apart completes a group's sum (the fused review pooling of the state sweep).
template <int Q, int COLS, int NT, bool GROUPED = false>
struct Rows {
    static constexpr int UPR = COLS / 8;
    static constexpr int PER = Q * UPR / NT;
    static_assert(Q * UPR % NT == 0, "tile must split evenly over the workgroup");
    static_assert(!GROUPED || (UPR == 8 && PER == 4 && NT == 256), "grouped rows: 64 columns, 128 rows, 256 threads");
    u32x4 r[PER];

    __device__ __forceinline__ static int row_of(int it)
    {
        if constexpr (GROUPED) {
            const int lane = threadIdx.x & 63, r8 = lane >> 3;
            return 8 * (4 * (int)(threadIdx.x >> 6) + (r8 >> 1)) + 2 * it + (r8 & 1);
        } else {
            return (threadIdx.x + NT * it) / UPR;
        }
    }
    __device__ __forceinline__ static int cc_of(int it) { return (threadIdx.x + NT * it) % UPR; }

    __device__ __forceinline__ void load(const __bf16 *base, size_t row_stride, const uint32_t *srow,
                                         size_t batch_rows)
    {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const uint32_t row = srow[row_of(it)];
            r[it] = *(const u32x4 *)(base + (batch_rows + (row != ~0u ? row : 0u)) * row_stride + 8 * cc_of(it));
        }
    }
    // load with streaming (non-temporal) loads: for rows read once per sweep, so that they do
    // not push data that other workgroups reuse out of L2
    __device__ __forceinline__ void load_nt(const __bf16 *base, size_t row_stride, const uint32_t *srow,
                                            size_t batch_rows)
    {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const uint32_t row = srow[row_of(it)];
            r[it] = __builtin_nontemporal_load(
                (const u32x4 *)(base + (batch_rows + (row != ~0u ? row : 0u)) * row_stride + 8 * cc_of(it)));
        }
    }
    template <int LD>
    __device__ __forceinline__ void store(__bf16 *dst) const
    {
#pragma unroll
        for (int it = 0; it < PER; ++it) *(u32x4 *)(dst + row_of(it) * LD + 8 * cc_of(it)) = r[it];
    }
    // bf16 -> fp16 (exact for values inside the fp16 normal range)
    template <int LD>
    __device__ __forceinline__ void store_f16(__bf16 *dst) const
    {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack2h(lo_f(r[it][e]), hi_f(r[it][e]));
            *(u32x4 *)(dst + row_of(it) * LD + 8 * cc_of(it)) = o;
        }
    }
    // store_f16 with the thread index passed in (t = threadIdx.x)
    template <int LD>
    __device__ __forceinline__ void store_f16_at(__bf16 *dst, int t) const
    {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack2h(lo_f(r[it][e]), hi_f(r[it][e]));
            const int k = t + NT * it;
            *(u32x4 *)(dst + (k / UPR) * LD + 8 * (k % UPR)) = o;
        }
    }
    template <int LD>
    __device__ __forceinline__ void store_scaled(__bf16 *dst, int it, float w) const
    {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack2(lo_f(r[it][e]) * w, hi_f(r[it][e]) * w);
        *(u32x4 *)(dst + row_of(it) * LD + 8 * cc_of(it)) = o;
    }
};

// Global row of sequence position i (< L): through the permutation table, or
// the identity when there is none; ~0u past the end.
__device__ __forceinline__ uint32_t seq_row(const uint32_t *perm, uint32_t i, uint32_t L)
{
    return i < L ? (perm ? perm[i] : i) : ~0u;
}

// Stored local backward states (P x S per chunk) are kept in accumulator order: 16-byte piece k holds
// the 8 values of accumulator registers 8q..8q+7 of lane l of the 32x32 tile (s-block sb, p-block pt)
// of G^T, k = ((sb * 2 + pt) * 2 + q) * 64 + l. Those are p = 32 pt + l % 32 and two runs of 4
// consecutive s starting at s_a = 32 sb + 16 q + 4 (l / 32) and s_a + 8.
struct HbPiece {
    int p, s_a;
};
__device__ __forceinline__ HbPiece hb_piece(int k)
{
    const int l = k & 63, q = (k >> 6) & 1, t = k >> 7;
    return {32 * (t & 1) + (l & 31), 32 * (t >> 1) + 16 * q + 4 * (l >> 5)};
}

// Operands in MFMA operand order: block blk (a 32-row block of the operand's m or n index) and k-block kb
// (16 consecutive values of the contraction index, kblocks of them per block) hold, for lane l, the 8
// values of row 32 blk + l % 32 at k = 16 kb + 8 (l / 32) + 0..7, as the l-th 16 bytes of a 1 KB piece.
// Returns the element offset of that lane's 8 values.
__device__ __forceinline__ int op_piece(int blk, int kb, int kblocks, int l)
{
    return ((blk * kblocks + kb) * 64 + l) * 8;
}

// ---------------------------------------------------------------------------
// 0. RMS permutation table: perm[i] = canonical token of scan position i.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_perm(uint32_t *__restrict__ perm, uint32_t N, int order, uint32_t T,
                                              uint32_t H, uint32_t W)
{
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i < N) perm[i] = rms_index32(i, order, T, H, W);
}

// ---------------------------------------------------------------------------
// 1a. Right-to-left sweep of the review sequence (pooled rows in order, B pooled bf16): segment
// summaries only. grid = 8 * ceil(batch * nheads / 8); one segment per head.
// Each wave owns (s-block, p-block) tile pairs: the backward state G^T and the forward sum F^T of the
// same tile share both operand tiles, B^T and x (fp16); the per-token weights of the two sums,
// dt exp(ce) and dt exp(tot - cs + logD), are applied to the x operand in registers (packed fp16).
// The x and B rows and per-token values of the chunk two to the left are loaded every step (clamped at
// the segment start), so the compiler's memory waits are not widened by paths that skip them.
// ---------------------------------------------------------------------------
template <int S, int Q>
__global__ __launch_bounds__(Q * 4) void k_states_review(const __bf16 *__restrict__ x, const __bf16 *__restrict__ Bm,
                                                         const float *__restrict__ dtT, const float *__restrict__ csT,
                                                         const float *__restrict__ A, float *__restrict__ segF,
                                                         float *__restrict__ segB, float *__restrict__ segA,
                                                         int nheads, int G, uint32_t L, uint32_t Lpad, int nch,
                                                         int segch, int nseg, int seg_base, int nseg_total,
                                                         uint32_t total_items)
{
    constexpr int NT = Q * 4, NW = Q / 16;          // Q/16 waves, two per SIMD at Q = 128
    constexpr int LX = P + XPAD, LB = S + XPAD;
    constexpr int PAIRS = S / 16;                   // tile pairs: (S/32 s-blocks) x (2 p-blocks)
    constexpr int TP = PAIRS >= NW ? PAIRS / NW : 1;
    constexpr int BPER = Q * S / 8 / NT;            // 16-byte pieces of the B tile per thread
    __shared__ _Float16 xn[Q * LX];   // x (fp16)
    __shared__ _Float16 bn[Q * LB];   // B (fp16)
    __shared__ __attribute__((aligned(16))) _Float16 s_wb[Q], s_wf[Q];  // per-token weights
    __shared__ uint32_t s_row[Q];     // global rows of the next chunk to fetch

    const uint32_t item = xcd_item();
    if (item >= total_items) return;
    const int h = item % nheads;
    const uint32_t rest = item / nheads;
    const int seg = rest % nseg, b = rest / nseg;
    const int g = h / (nheads / G);
    const int c_lo = seg * segch, c_hi = min(nch, c_lo + segch);

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool active = PAIRS >= NW || wave * TP < PAIRS;  // every wave when there are enough pairs
    const bool row_thread = wave < Q / 64;  // tid < Q: owns one row-table entry and one token's weights
    f32x16 accG[TP], accF[TP];
#pragma unroll
    for (int i = 0; i < TP; ++i) accG[i] = accF[i] = f32x16{};

    const float a = A[h];
    const size_t bh = (size_t)b * nheads + h;
    const size_t drow = bh * Lpad;
    // x and B rows and per-token values are fetched two chunks ahead into two alternating register
    // stages (their latency exceeds a chunk's work).
    struct Stage {
        Rows<Q, P, NT> xr;
        u32x4 bq[BPER];  // B pieces k = tid + NT it (row k / (S / 8), 8 columns at 8 (k % (S / 8)))
        float tok_d, tok_c, tot;
    };
    Stage stA, stB;
    uint32_t pnext = 0u;  // row-table entry of the chunk after the one fetched last
    bool pvalid = false;
    auto fetch = [&](Stage &stg, int c) {
        const int tq = tid & (Q - 1);
        const uint32_t i = (uint32_t)(c - 1) * Q + tq;
        pvalid = c > c_lo && i < L;
        pnext = i;
        stg.xr.load(x + (size_t)h * P, (size_t)nheads * P, s_row, (size_t)b * L);
        Rows<Q, S, NT> br;
        br.load(Bm + (size_t)g * S, (size_t)G * S, s_row, (size_t)b * L);
#pragma unroll
        for (int it = 0; it < BPER; ++it) stg.bq[it] = br.r[it];
        const size_t crow0 = drow + (size_t)c * Q;
        stg.tok_d = dtT[crow0 + tq];
        stg.tok_c = csT[crow0 + tq];
        stg.tot = csT[crow0 + Q - 1];
    };
    // Prologue: rows and data of the rightmost chunk, then the rows and x of the one before.
    if (row_thread) s_row[tid] = seq_row(nullptr, (uint32_t)(c_hi - 1) * Q + tid, L);
    __syncthreads();
    fetch(stA, c_hi - 1);
    __syncthreads();  // every lane has read the rows of chunk c_hi - 1
    s_row[tid & (Q - 1)] = pvalid ? pnext : ~0u;
    __syncthreads();
    fetch(stB, max(c_hi - 2, c_lo));  // a one-chunk segment: issued, unused
    float logD = 0.f;  // sum of dt*A over the chunks right of the current one

    auto step = [&](Stage &cur, int c) {
        __syncthreads();  // previous chunk's MFMA reads of LDS and the row-table reads are done
        // The staged values are used from here on (their loads had two steps to complete).
#pragma unroll
        for (int it = 0; it < Rows<Q, P, NT>::PER; ++it) pin(cur.xr.r[it]);
#pragma unroll
        for (int it = 0; it < BPER; ++it) pin(cur.bq[it]);
        pin(cur.tok_d);
        pin(cur.tok_c);
        pin(cur.tot);
        pin(pnext);
        const float tot_c = cur.tot;
        cur.xr.template store_f16<LX>((__bf16 *)xn);
#pragma unroll
        for (int it = 0; it < BPER; ++it) {
            const int k = tid + NT * it;
            u32x4 v = cur.bq[it];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = pack2h(lo_f(v[e]), hi_f(v[e]));
            *(u32x4 *)&bn[(k / (S / 8)) * LB + 8 * (k % (S / 8))] = v;
        }
        if (row_thread) {
            const float d = cur.tok_d, cs = cur.tok_c;
            s_wb[tid] = (_Float16)(d * ex2((cs - d * a) * LOG2E));
            s_wf[tid] = (_Float16)(d * ex2((tot_c - cs + logD) * LOG2E));
        }
        // Rows of chunk c - 2. Every thread stores its (identical) entry: a use on all paths keeps
        // the row load where it is issued.
        s_row[tid & (Q - 1)] = pvalid ? pnext : ~0u;
        __syncthreads();

        fetch(cur, max(c - 2, c_lo));  // near the segment start: issued, unused
        if (active) {
            const float dec = ex2(tot_c * LOG2E);
#pragma unroll
            for (int i = 0; i < TP; ++i) accG[i] *= dec;
#pragma unroll
            for (int kb = 0; kb < Q / 16; ++kb) {
                const f16x8 wb8 = *(const f16x8 *)(s_wb + 16 * kb + 8 * half);
                const f16x8 wf8 = *(const f16x8 *)(s_wf + 16 * kb + 8 * half);
#pragma unroll
                for (int i = 0; i < TP; ++i) {
                    const int j = wave * TP + i;
                    const f16x8 af = __builtin_bit_cast(f16x8, frag_tr((const __bf16 *)bn, LB, 16 * kb, 32 * (j >> 1)));
                    const f16x8 xv = __builtin_bit_cast(f16x8, frag_tr((const __bf16 *)xn, LX, 16 * kb, 32 * (j & 1)));
                    accG[i] = mfma16(af, xv * wb8, accG[i]);
                    accF[i] = mfma16(af, xv * wf8, accF[i]);
                }
            }
        }
        logD += tot_c;
    };
    int c = c_hi - 1;
    for (; c - 1 >= c_lo; c -= 2) {
        step(stA, c);
        step(stB, c - 1);
    }
    if (c >= c_lo) step(stA, c);

    // Segment summaries: G (backward state entering the segment from its right end, from zero) and F.
    if (active) {
        const int col = lane & 31;
        float *dG = segB + (bh * nseg_total + seg_base + seg) * (size_t)(P * S);
        float *dF = segF + (bh * nseg_total + seg_base + seg) * (size_t)(P * S);
#pragma unroll
        for (int i = 0; i < TP; ++i) {
            const int j = wave * TP + i, sb = j >> 1, pb = j & 1;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const size_t o = (size_t)(32 * pb + col) * S + 32 * sb + 8 * g4 + 4 * half;
                *(f32x4 *)(dG + o) = f32x4{accG[i][4 * g4], accG[i][4 * g4 + 1], accG[i][4 * g4 + 2], accG[i][4 * g4 + 3]};
                *(f32x4 *)(dF + o) = f32x4{accF[i][4 * g4], accF[i][4 * g4 + 1], accF[i][4 * g4 + 2], accF[i][4 * g4 + 3]};
            }
        }
    }
    if (tid == 0) segA[bh * nseg_total + seg_base + seg] = logD;
}

// ---------------------------------------------------------------------------
// 2. States at segment borders. grid (ceil(P*S / 256), nheads, batch).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_seg_pass(const float *__restrict__ segF, const float *__restrict__ segB,
                                                  const float *__restrict__ segA, float *__restrict__ hinF,
                                                  __bf16 *__restrict__ hinB, int PS, int nseg, int nseg_total,
                                                  int has_review)
{
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= PS) return;
    const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
    const float *F = segF + bh * nseg_total * PS + e;
    const float *Bk = segB + bh * nseg_total * PS + e;
    const float *sa = segA + bh * nseg_total;
    // Unrolled so that the summary loads of several segments (independent of the carried
    // state) are in flight together.
    float run = has_review ? F[(size_t)nseg * PS] : 0.f;
#pragma unroll 8
    for (int j = 0; j < nseg; ++j) {
        hinF[(bh * nseg + j) * PS + e] = run;
        run = ex2(sa[j] * LOG2E) * run + F[(size_t)j * PS];
    }
    run = has_review ? Bk[(size_t)nseg * PS] : 0.f;
#pragma unroll 8
    for (int j = nseg - 1; j >= 0; --j) {
        hinB[(bh * nseg + j) * PS + e] = (__bf16)run;
        run = ex2(sa[j] * LOG2E) * run + Bk[(size_t)j * PS];
    }
}

// ---------------------------------------------------------------------------
// 3. Per chunk and group (grid (nch, G, batch)), the sweeps' operands in MFMA operand order (see
//    op_piece), so that each wave reads each operand with one contiguous 1 KB load per k-block:
//    cb    CB[t][u] = C_t . B_u (fp16), token block tb = t / 32, k-blocks over u;
//    cfrag C rows (bf16), token block tb, k-blocks over the state index s;
//    bfrag B^T rows (fp16), state block sb = s / 32, k-blocks over u.
// The chunk's B and C rows are gathered once into LDS (B also as fp16 at the stride of the
// transposing read); CB is computed as CB^T = B C^T so each lane holds 4 consecutive u of one t.
// ---------------------------------------------------------------------------
template <int S, int Q>
__global__ __launch_bounds__(NT) void k_cb(const __bf16 *__restrict__ Bm, const __bf16 *__restrict__ Cm,
                                           const uint32_t *__restrict__ perm, _Float16 *__restrict__ cb,
                                           __bf16 *__restrict__ cfrag, _Float16 *__restrict__ bfrag, int G, uint32_t L)
{
    constexpr int LR = S + 8;     // row stride of the row-read tiles (conflict-free 16-byte reads)
    constexpr int LT = S + XPAD;  // row stride of the fp16 B tile (conflict-free transposing reads)
    __shared__ __attribute__((aligned(16))) __bf16 bs[Q * LR];
    __shared__ __attribute__((aligned(16))) __bf16 cs[Q * LR];
    __shared__ __attribute__((aligned(16))) _Float16 bt[Q * LT];
    __shared__ uint32_t srow[Q];
    const uint32_t c = blockIdx.x;
    const int g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int TB = Q / 32, KU = Q / 16, KS = S / 16;
    const size_t rs = (size_t)G * S;
    const size_t chunk = ((size_t)b * G + g) * gridDim.x + c;

    for (int u = tid; u < Q; u += NT) srow[u] = seq_row(perm, c * Q + u, L);
    __syncthreads();
    // B and C rows, 16-byte pieces; a position past the end holds zeros.
    constexpr int PER = Q * S / 8 / NT;
    static_assert(Q * S / 8 % NT == 0, "pieces must split evenly");
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int k = tid + NT * it, row = k / (S / 8), c8 = k % (S / 8);
        const uint32_t r = srow[row];
        const size_t off = ((size_t)b * L + (r != ~0u ? r : 0u)) * rs + (size_t)g * S + 8 * c8;
        u32x4 vb = *(const u32x4 *)(Bm + off), vc = *(const u32x4 *)(Cm + off);
        if (r == ~0u) vb = vc = u32x4{0, 0, 0, 0};
        *(u32x4 *)(bs + row * LR + 8 * c8) = vb;
        *(u32x4 *)(cs + row * LR + 8 * c8) = vc;
        u32x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = pack2h(lo_f(vb[e]), hi_f(vb[e]));
        *(u32x4 *)(bt + row * LT + 8 * c8) = h;
    }
    __syncthreads();

    _Float16 *out = cb + chunk * (size_t)(Q * Q);
    constexpr int TILES = TB * TB / 4;  // per wave
#pragma unroll
    for (int k = 0; k < TILES; ++k) {
        const int ti = wave + 4 * k;
        const int ub = ti / TB, tb = ti % TB;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kb = 0; kb < KS; ++kb)
            acc = mfma(frag_rm(bs, LR, 32 * ub, 16 * kb), frag_rm(cs, LR, 32 * tb, 16 * kb), acc);
        // acc: rows u = 32 ub + 8 g4 + 4 half + j, column t = 32 tb + col. The 8-value piece holding
        // u = 32 ub + 8 g4 + 0..7 is k-block 2 ub + g4 / 2, lane col + 32 (g4 % 2).
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            f16x4 v4;
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] = (_Float16)acc[4 * g4 + j];
            *(f16x4 *)(out + op_piece(tb, 2 * ub + (g4 >> 1), KU, col + 32 * (g4 & 1)) + 4 * half) = v4;
        }
    }
    // C pieces: block (token block tb, k-block kb over s); B^T pieces: block (state block sb, k-block
    // kb over u), lane l holding B[16 kb + 8 (l / 32) + 0..7][32 sb + l % 32].
    __bf16 *co = cfrag + chunk * (size_t)(Q * S);
    _Float16 *bfo = bfrag + chunk * (size_t)(Q * S);
    constexpr int BLOCKS = TB * KS;  // = (S / 32) * KU
    static_assert(BLOCKS % 4 == 0, "blocks must split evenly over the waves");
#pragma unroll
    for (int k = 0; k < BLOCKS / 4; ++k) {
        const int blk = wave + 4 * k;
        const int tb = blk / KS, kb = blk % KS;
        *(bf16x8 *)(co + op_piece(tb, kb, KS, lane)) = frag_rm(cs, LR, 32 * tb, 16 * kb);
        const int sb = blk / KU, kbu = blk % KU;
        *(bf16x8 *)(bfo + op_piece(sb, kbu, KU, lane)) = frag_tr((const __bf16 *)bt, LT, 16 * kbu, 32 * sb);
    }
}

// ---------------------------------------------------------------------------
// 1b. Right-to-left sweep of the main sequence: the backward state entering every chunk from the right
// (stored as bf16 for the output sweep) and the segment summaries G, F and sum(dt A).
// grid = 8 * ceil(batch * nseg * nheads / 8); item = (b * nseg + seg) * nheads + h.
// Workgroups of four waves, two per CU. B^T comes from L2 in MFMA operand order (bfrag, one
// chunk ahead in two alternating register sets) and only x passes through LDS. Wave w owns the G^T
// and F^T tiles of state block s-block(w) (both p-blocks at S = 128); the per-token weights of the two
// sums are applied to the B^T operand, so one scaled operand serves both p-blocks. x rows and
// per-token values come two chunks ahead through two register stages.
// ---------------------------------------------------------------------------
// POOL: the review pooling of x is fused into the sweep. Every aligned group of 8 consecutive scan
// positions lies in one pool block (the scan's fastest axis has a pool extent that is a multiple of 8), so
// the sweep sums each group's x rows (fp32, rounded to bf16) into xpart[b][run][head][P], run = the group's
// index along that axis; k_pool_runs then averages the runs of each pool block. x is read once for both.
template <int S, int Q, bool POOL>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
void k_states(const __bf16 *__restrict__ x, const _Float16 *__restrict__ bfrag, const uint32_t *__restrict__ perm,
               const float *__restrict__ dtT, const float *__restrict__ csT, const float *__restrict__ A,
               __bf16 *__restrict__ hb_local, float *__restrict__ delta, float *__restrict__ segF,
               float *__restrict__ segB, float *__restrict__ segA, __bf16 *__restrict__ xpart, uint32_t run_stride,
               uint32_t nrun, int nheads, int G, uint32_t L, uint32_t Lpad, int nch, int segch, int nseg,
               int nseg_total, uint32_t total_items)
{
    constexpr int LX = P + XPAD;
    constexpr int KU = Q / 16;  // k-blocks over the chunk's tokens
    constexpr int TT = S / 64;  // G^T (and F^T) tiles per wave: state block sb, p-blocks pb0 ..
    __shared__ _Float16 xn[Q * LX];  // x (fp16)
    __shared__ __attribute__((aligned(16))) _Float16 s_wb[Q], s_wf[Q];  // per-token weights
    __shared__ uint32_t s_row[Q];    // global rows of the next chunk to fetch

    const uint32_t item = xcd_item();
    if (item >= total_items) return;
    const int h = item % nheads;
    const uint32_t rest = item / nheads;
    const int seg = rest % nseg, b = rest / nseg;
    const int g = h / (nheads / G);
    const int c_lo = seg * segch, c_hi = min(nch, c_lo + segch);

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool row_thread = tid < Q;
    const int sb = (wave * TT) >> 1, pb0 = (wave * TT) & 1;
    f32x16 accG[TT], accF[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) accG[i] = accF[i] = f32x16{};

    const float a = A[h];
    const size_t bh = (size_t)b * nheads + h;
    const size_t drow = bh * Lpad;
    const size_t gch = ((size_t)b * G + g) * nch;
    using XRows = Rows<Q, P, NT, POOL>;
    struct Stage {
        XRows xr;
        float tok_d, tok_c, tot;
        uint32_t prow;  // POOL: canonical token of this thread's first row (~0u past the end)
    };
    Stage stA, stB;
    u32x4 bA[KU], bB[KU];  // B^T operands of the chunk being summed and of the next one
    uint32_t pnext = 0u;   // row-table entry of the chunk after the one fetched last
    bool pvalid = false;
    auto fetch = [&](Stage &stg, int c) {
        // The row-table load first: a wait for it then covers only older loads.
        const int tq = tid & (Q - 1);
        const uint32_t i = (uint32_t)(c - 1) * Q + tq;
        pvalid = c > c_lo && i < L;
        pnext = perm[pvalid ? i : 0u];  // selected against pvalid where it is stored
        stg.xr.load_nt(x + (size_t)h * P, (size_t)nheads * P, s_row, (size_t)b * L);
        if constexpr (POOL) stg.prow = s_row[XRows::row_of(0)];
        const size_t crow0 = drow + (size_t)c * Q;
        stg.tok_d = dtT[crow0 + tq];
        stg.tok_c = csT[crow0 + tq];
        stg.tot = csT[crow0 + Q - 1];
    };
    auto fetch_b = [&](u32x4 (&bq)[KU], int c) {
        const _Float16 *src = bfrag + (gch + c) * (size_t)(Q * S) + op_piece(sb, 0, KU, lane);
#pragma unroll
        for (int kb = 0; kb < KU; ++kb) bq[kb] = *(const u32x4 *)(src + 512 * kb);
    };
    // Prologue: rows and data of the rightmost chunk, then the rows and x of the one before.
    if (row_thread) s_row[tid] = seq_row(perm, (uint32_t)(c_hi - 1) * Q + tid, L);
    __syncthreads();
    fetch(stA, c_hi - 1);
    fetch_b(bA, c_hi - 1);
    __syncthreads();  // every lane has read the rows of chunk c_hi - 1
    s_row[tid & (Q - 1)] = pvalid ? pnext : ~0u;
    __syncthreads();
    fetch(stB, max(c_hi - 2, c_lo));  // a one-chunk segment: issued, unused
    float logD = 0.f;  // sum of dt*A over the chunks right of the current one

    auto step = [&](Stage &cur, u32x4 (&bc)[KU], u32x4 (&bn)[KU], int c) {
        // Backward state entering chunk c from the right, in accumulator order (see hb_piece): packed
        // now, stored once the chunk's first MFMAs are issued.
        bf16x8 hbv[TT][2];
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e) hbv[i][q][e] = (__bf16)accG[i][8 * q + e];
        auto store_hb = [&]() {
            __bf16 *dst = hb_local + (bh * nch + c) * (size_t)(P * S);
#pragma unroll
            for (int i = 0; i < TT; ++i)
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    __builtin_nontemporal_store(hbv[i][q], (bf16x8 *)(dst + (((wave * TT + i) * 2 + q) * 64 + lane) * 8));
            delta[bh * nch + c] = ex2(logD * LOG2E);  // every thread writes the same value
        };

        __syncthreads();  // previous chunk's reads of xn and the row-table reads are done
        // The staged values are used from here on (their loads had two steps to complete).
#pragma unroll
        for (int it = 0; it < XRows::PER; ++it) pin(cur.xr.r[it]);
        pin(cur.tok_d);
        pin(cur.tok_c);
        pin(cur.tot);
        pin(pnext);
        const float tot_c = cur.tot;
        cur.xr.template store_f16<LX>((__bf16 *)xn);
        if constexpr (POOL) {
            // This thread's four rows of its group, then the lane 8 apart holds the group's other four.
            float acc[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] = lo_f(cur.xr.r[0][e]);
                acc[2 * e + 1] = hi_f(cur.xr.r[0][e]);
            }
#pragma unroll
            for (int it = 1; it < 4; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += lo_f(cur.xr.r[it][e]);
                    acc[2 * e + 1] += hi_f(cur.xr.r[it][e]);
                }
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += dpp_ror8(acc[e]);
            pin(cur.prow);
            const uint32_t n = cur.prow;
            if (!(lane & 8) && n != ~0u) {
                const size_t run = (size_t)(n / (8u * run_stride)) * run_stride + n % run_stride;
                bf16x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (__bf16)acc[e];
                __builtin_nontemporal_store(
                    v, (bf16x8 *)(xpart + (((size_t)b * nrun + run) * nheads + h) * P + 8 * (lane & 7)));
            }
        }
        if (row_thread) {
            const float d = cur.tok_d, cs = cur.tok_c;
            s_wb[tid] = (_Float16)(d * ex2((cs - d * a) * LOG2E));
            s_wf[tid] = (_Float16)(d * ex2((tot_c - cs + logD) * LOG2E));
        }
        // Rows of chunk c - 2. Every thread stores its (identical) entry: a use on all paths keeps
        // the row load where it is issued.
        s_row[tid & (Q - 1)] = pvalid ? pnext : ~0u;
        __syncthreads();

        const float dec = ex2(tot_c * LOG2E);
#pragma unroll
        for (int i = 0; i < TT; ++i) accG[i] *= dec;
#pragma unroll
        for (int kb = 0; kb < KU; ++kb) {
            const f16x8 wb8 = *(const f16x8 *)(s_wb + 16 * kb + 8 * half);
            const f16x8 wf8 = *(const f16x8 *)(s_wf + 16 * kb + 8 * half);
            const f16x8 af = __builtin_bit_cast(f16x8, bc[kb]);
            const f16x8 afb = af * wb8, aff = af * wf8;
#pragma unroll
            for (int i = 0; i < TT; ++i) {
                const f16x8 xv = __builtin_bit_cast(f16x8, frag_tr((const __bf16 *)xn, LX, 16 * kb, 32 * (pb0 + i)));
                accG[i] = mfma16(afb, xv, accG[i]);
                accF[i] = mfma16(aff, xv, accF[i]);
            }
            // The next loads issue while this chunk's MFMAs run (a load waiting for the memory pipeline
            // holds up only what this wave issues after it): B (needed next step) before x (needed in
            // two), so that waits complete in issue order.
            if (kb == 0) store_hb();
            if (kb == 1) fetch_b(bn, max(c - 1, c_lo));
            if (kb == 3) fetch(cur, max(c - 2, c_lo));  // near the segment start: issued, unused
        }
        logD += tot_c;
    };
    int c = c_hi - 1;
    for (; c - 1 >= c_lo; c -= 2) {
        step(stA, bA, bB, c);
        step(stB, bB, bA, c - 1);
    }
    if (c >= c_lo) step(stA, bA, bB, c);

    // Segment summaries: G (backward state entering the segment from its right end, from zero) and F.
    {
        float *dG = segB + (bh * nseg_total + seg) * (size_t)(P * S);
        float *dF = segF + (bh * nseg_total + seg) * (size_t)(P * S);
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            const int pb = pb0 + i;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const size_t o = (size_t)(32 * pb + col) * S + 32 * sb + 8 * g4 + 4 * half;
                *(f32x4 *)(dG + o) = f32x4{accG[i][4 * g4], accG[i][4 * g4 + 1], accG[i][4 * g4 + 2], accG[i][4 * g4 + 3]};
                *(f32x4 *)(dF + o) = f32x4{accF[i][4 * g4], accF[i][4 * g4 + 1], accF[i][4 * g4 + 2], accF[i][4 * g4 + 3]};
            }
        }
    }
    if (tid == 0) segA[bh * nseg_total + seg] = logD;
}

// ---------------------------------------------------------------------------
// 4. Left-to-right output sweep. Same items as k_states (main segments); workgroups of four waves (one
// per SIMD) and two workgroups per CU, so that the phases of one overlap those of the other.
//
// Per chunk, two phases separated by barriers:
//   compute  The operands with a single consumer come from global memory in operand order (B^T, CB, C;
//            group data that the heads of a group share in L2), so only x and the two states pass
//            through LDS. Wave w owns the Y^T tiles of one token block (both p-blocks at Q = 128) and the
//            Hf^T tiles of one state block. Per 16-token k-block, the x operands (transposed LDS reads)
//            serve both the intra-chunk product X^T M^T (fp16) and the state update
//            Hf^T = exp(tot) Hf^T + B^T (w x)^T (w = dt exp(tot - cs) applied to the x operand in
//            registers); each lane builds its M^T operand (row t = its token, 8 consecutive u) from its
//            CB piece in registers. Then the inter-chunk terms ef (Hf C^T) + eb (Hb C^T) are added with
//            ef = exp(cs), eb = exp(tot - ce) per token, and Y goes to LDS as bf16 rows.
//   store    Y rows leave as contiguous 16-byte pieces; the next chunk is staged: x (fp16), the forward
//            state Hf (from the accumulators), the backward state Hb = stored local state + decay *
//            border state, and the per-token decay data.
// Every load and store in the loop is unconditional (a lane past the end of the sequence reads row 0
// and stores into a scratch row), and no load result crosses the loop edge, so the compiler's memory
// waits stay exact.
// ---------------------------------------------------------------------------
template <int S, int Q>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
void k_out(const __bf16 *__restrict__ x, const _Float16 *__restrict__ bfrag, const __bf16 *__restrict__ cfrag,
           const _Float16 *__restrict__ cb, const uint32_t *__restrict__ perm, const float *__restrict__ dtT,
           const float *__restrict__ csT, const float *__restrict__ A, const float *__restrict__ Dv,
           const __bf16 *__restrict__ hb_local, const float *__restrict__ delta, const float *__restrict__ hinF,
           const __bf16 *__restrict__ hinB, __bf16 *__restrict__ y, __bf16 *__restrict__ ytrash, int nheads, int G,
           uint32_t N, uint32_t Lpad, int nch, int segch, int nseg, uint32_t total_items)
{
    constexpr int LX = P + XPAD, SS = S + 8, LY = P + 8;
    constexpr int KU = Q / 16;  // k-blocks over the chunk's tokens
    constexpr int KS = S / 16;  // k-blocks over the state
    constexpr int YT = Q / 64;  // Y^T tiles per wave: token block tb, p-blocks pb0 ..
    constexpr int HT = S / 64;  // Hf^T tiles per wave: state block hsb, p-blocks hpb0 ..
    constexpr int NPX = (YT == 2 || HT == 2) ? 2 : 1;  // p-blocks of the x operands a wave reads
    __shared__ _Float16 xn[Q * LX];  // x as fp16: operand of the intra-chunk product and of the state update
    __shared__ __bf16 hfl[P * SS];   // forward state entering the chunk, [p][s]
    __shared__ __bf16 hbl[P * SS];   // backward state entering the chunk from the right, [p][s]
    __shared__ __attribute__((aligned(16))) __bf16 ybuf[Q * LY];  // output rows [t][p]
    // per token: cs, ce (log2 units), dt, the split decay factors of the off-diagonal blocks, the state weight
    __shared__ __attribute__((aligned(16))) float s_cs[Q], s_ce[Q], s_dt[Q];
    __shared__ __attribute__((aligned(16))) _Float16 s_gl[Q], s_gu[Q], s_w[Q];
    __shared__ uint32_t s_row[Q];    // global rows of the chunk after the staged one
    __shared__ uint32_t s_rowy[Q];   // global rows of the chunk whose output is in ybuf

    const uint32_t item = xcd_item();
    if (item >= total_items) return;
    const int h = item % nheads;
    const uint32_t rest = item / nheads;
    const int seg = rest % nseg, b = rest / nseg;
    const int g = h / (nheads / G);
    const int c_lo = seg * segch, c_hi = min(nch, c_lo + segch);
    const size_t bh = (size_t)b * nheads + h;
    const size_t drow = bh * Lpad;

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool row_thread = tid < Q;
    const int tb = (wave * YT) >> 1, pb0 = (wave * YT) & 1;
    const int hsb = (wave * HT) >> 1, hpb0 = (wave * HT) & 1;
    const int px0 = NPX == 2 ? 0 : (wave & 1);  // with one p-block each, pb0 = hpb0 = wave % 2
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
    // Border state of the backward direction (bf16), for this thread's staging pieces (in the stored
    // states' accumulator order; see hb_piece). It is the same for the whole segment and L2-resident;
    // it is reloaded before each staging rather than held in registers through the compute phase (the
    // pinned offset keeps the compiler from hoisting the loads out of the loop).
    constexpr int HBC = PS / 8 / NT;
    u32x4 hinb[HBC];
    const size_t hinb_off = (bh * nseg + seg) * (size_t)PS;
    auto load_hinb = [&]() {
        size_t off = hinb_off;
        asm volatile("" : "+s"(off));
        const __bf16 *hs = hinB + off;
#pragma unroll
        for (int it = 0; it < HBC; ++it) {
            const HbPiece pc = hb_piece(tid + NT * it);
            const u32x2 lo = *(const u32x2 *)(hs + pc.p * S + pc.s_a);
            const u32x2 hi = *(const u32x2 *)(hs + pc.p * S + pc.s_a + 8);
            hinb[it] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };

    Rows<Q, P, NT> xr;
    const size_t gch = ((size_t)b * G + g) * nch;  // chunk index base of this group
    const int t_tok = 32 * tb + col;  // this lane's token inside the chunk (Y^T column)

    // Per-head data of the next chunk (HBM): loaded during the compute phase, consumed by the staging
    // at the end of the same iteration.
    u32x4 hbr[HBC];
    float tok_d = 0.f, tok_c = 0.f, tot = 0.f, dl = 0.f;
    uint32_t pnext = 0u;
    bool pvalid = false;
    auto fetch = [&](int c) {
        // x rows and stored states are read once: streaming loads keep the group operands and
        // border states that other workgroups reuse in L2
        xr.load_nt(x + (size_t)h * P, (size_t)nheads * P, s_row, (size_t)b * N);
        const __bf16 *src = hb_local + (bh * nch + c) * (size_t)PS;
#pragma unroll
        for (int it = 0; it < HBC; ++it) hbr[it] = __builtin_nontemporal_load((const u32x4 *)(src + 8 * (tid + NT * it)));
        // Every thread issues the same loads; the per-token values matter for tid < Q only.
        const int tq = tid & (Q - 1);
        const size_t crow0 = drow + (size_t)c * Q;
        tok_d = dtT[crow0 + tq];
        tok_c = csT[crow0 + tq];
        {
            const uint32_t i = (uint32_t)(c + 1) * Q + tq;
            pvalid = c + 1 < c_hi && i < N;
            pnext = perm[pvalid ? i : 0u];  // selected against pvalid where it is stored
        }
        tot = csT[crow0 + Q - 1];
        dl = delta[bh * nch + c];
    };
    uint32_t rowc = 0u;  // row-thread: global row of token tid of the staged chunk (~0u past the end)
    // The staging and output addresses come from a thread index pinned where they are used, so the
    // compiler recomputes them per chunk rather than holding them (and spilling them) across the loop.
    auto stage = [&]() {
        int pt = tid;
        pin(pt);
        pt &= NT - 1;  // lets the compiler fold the per-iteration offsets into immediates
        const int pcol = pt & 31, phalf = (pt >> 5) & 1;
        xr.template store_f16_at<LX>((__bf16 *)xn, pt);
#pragma unroll
        for (int i = 0; i < HT; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 v4;
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[j] = (__bf16)hacc[i][4 * g4 + j];
                *(bf16x4 *)&hfl[(32 * (hpb0 + i) + pcol) * SS + 32 * hsb + 8 * g4 + 4 * phalf] = v4;
            }
#pragma unroll
        for (int it = 0; it < HBC; ++it) {
            const HbPiece pc = hb_piece(pt + NT * it);
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack2(lo_f(hbr[it][e]) + dl * lo_f(hinb[it][e]), hi_f(hbr[it][e]) + dl * hi_f(hinb[it][e]));
            *(u32x2 *)&hbl[pc.p * SS + pc.s_a] = u32x2{o[0], o[1]};
            *(u32x2 *)&hbl[pc.p * SS + pc.s_a + 8] = u32x2{o[2], o[3]};
        }
        // Block-edge values of this token's 32-token block, from its lanes 0/31 (or 32/63).
        const int c0l = __builtin_amdgcn_readlane(__float_as_int(tok_c), 0);
        const int c31l = __builtin_amdgcn_readlane(__float_as_int(tok_c), 31);
        const int d0l = __builtin_amdgcn_readlane(__float_as_int(tok_d), 0);
        const int c0h = __builtin_amdgcn_readlane(__float_as_int(tok_c), 32);
        const int c31h = __builtin_amdgcn_readlane(__float_as_int(tok_c), 63);
        const int d0h = __builtin_amdgcn_readlane(__float_as_int(tok_d), 32);
        if (row_thread) {
            const float blk_cs0 = __int_as_float(half ? c0h : c0l);
            const float blk_cs_end = __int_as_float(half ? c31h : c31l);
            const float blk_dt0 = __int_as_float(half ? d0h : d0l);
            const float cs2 = tok_c * LOG2E, ce2 = (tok_c - tok_d * a) * LOG2E;
            s_dt[pt] = tok_d;
            s_cs[pt] = cs2;
            s_ce[pt] = ce2;
            // below-diagonal blocks: exp(cs_end - cs_u); above: exp(ce_u - ce_start); both <= 1
            s_gl[pt] = (_Float16)(tok_d * ex2(blk_cs_end * LOG2E - cs2));
            s_gu[pt] = (_Float16)(tok_d * ex2(ce2 - (blk_cs0 - blk_dt0 * a) * LOG2E));
            // weight of token u in the state carried out of the chunk
            s_w[pt] = (_Float16)(tok_d * ex2(tot * LOG2E - cs2));
            rowc = s_row[pt];
            s_row[pt] = pvalid ? pnext : ~0u;
        }
    };
    // Output rows of the chunk in ybuf: contiguous 16-byte pieces (a past-the-end row goes to scratch).
    // B^T (state update) and CB (intra-chunk product) of a chunk, per k-block in the order they are
    // consumed: group data that the heads of a group share in L2. The first half of the k-blocks is
    // loaded during the previous chunk, the second half at the start of the chunk.
    u32x4 bfr[KU], cbf[KU];
    auto fetch_group = [&](int c, int half_k) {
        const _Float16 *bs = bfrag + (gch + c) * (size_t)(Q * S) + op_piece(hsb, 0, KU, lane);
        const _Float16 *cs = cb + (gch + c) * (size_t)(Q * Q) + op_piece(tb, 0, KU, lane);
#pragma unroll
        for (int kb = half_k * (KU / 2); kb < (half_k + 1) * (KU / 2); ++kb) {
            bfr[kb] = *(const u32x4 *)(bs + 512 * kb);
            cbf[kb] = *(const u32x4 *)(cs + 512 * kb);
        }
    };
    auto store_y = [&]() {
        int pt = tid;
        pin(pt);
        pt &= NT - 1;  // lets the compiler fold the per-iteration offsets into immediates
#pragma unroll
        for (int it = 0; it < Q * (P / 8) / NT; ++it) {
            const int k = pt + NT * it;
            const int t = k / (P / 8), p8 = 8 * (k % (P / 8));
            const uint32_t r = s_rowy[t];
            __bf16 *dst = r != ~0u ? y + (((size_t)b * N + r) * nheads + h) * P + p8 : ytrash + p8;
            __builtin_nontemporal_store(*(const u32x4 *)&ybuf[t * LY + p8], (u32x4 *)dst);
        }
    };

    // Prologue: rows of the first chunk, its data, staged.
    if (row_thread) s_row[tid] = seq_row(perm, (uint32_t)c_lo * Q + tid, N);
    __syncthreads();
    fetch(c_lo);
    load_hinb();
    __syncthreads();
    stage();
    fetch_group(c_lo, 0);

    for (int c = c_lo; c < c_hi; ++c) {
        __syncthreads();  // staged chunk c visible

        const float tot_c = tot;
        const int cn = c + 1 < c_hi ? c + 1 : c;  // on the last iteration the loads are issued but unused
        // Load order within the chunk, so that every wait covers only older loads: the second half of
        // this chunk's B^T and CB; mid-loop, C of this chunk (inter-chunk terms, after the k-block
        // loop) and the next chunk's per-head data; after the inter-chunk terms, the border state
        // (staging) and the first half of the next chunk's B^T and CB.
        fetch_group(c, 1);
        u32x4 cfr[KS];
        const float cs_t = s_cs[t_tok], ce_t = s_ce[t_tok], dt_t = s_dt[t_tok];
        // position of this lane's token inside its diagonal pieces (pinned: recomputed per chunk
        // rather than held as hoisted per-element masks)
        int jd = col - 8 * half;
        pin(jd);
        {
            const float dec = ex2(tot_c * LOG2E);
#pragma unroll
            for (int i = 0; i < HT; ++i) hacc[i] *= dec;
        }
        // Per-lane factor of each off-diagonal 32-token block U of M, both <= 1: below the diagonal
        // block exp(cs_t - cs at the end of U), above it exp(ce at the start of U - ce_t).
        _Float16 fac[Q / 32];
#pragma unroll
        for (int U = 0; U < Q / 32; ++U)
            fac[U] = (_Float16)ex2(U < tb ? cs_t - s_cs[32 * U + 31] : s_ce[32 * U] - ce_t);
        f32x16 yacc[YT];
#pragma unroll
        for (int j = 0; j < YT; ++j) yacc[j] = f32x16{};
#pragma unroll
        for (int kb = 0; kb < KU; ++kb) {
            if (kb == KU / 2) {
                const __bf16 *src = cfrag + (gch + c) * (size_t)(Q * S) + op_piece(tb, 0, KS, lane);
#pragma unroll
                for (int k2 = 0; k2 < KS; ++k2) cfr[k2] = *(const u32x4 *)(src + 512 * k2);
                fetch(cn);
            }
            f16x8 xa[NPX];
#pragma unroll
            for (int i = 0; i < NPX; ++i)
                xa[i] = __builtin_bit_cast(f16x8, frag_tr((const __bf16 *)xn, LX, 16 * kb, 32 * (px0 + i)));
            // M^T operand: M[t_tok][u0 + 0..7]
            const int U = kb >> 1, u0 = 16 * kb + 8 * half;
            const f16x8 cb8 = __builtin_bit_cast(f16x8, cbf[kb]);
            f16x8 mf;
            if (U == tb) {
                const f32x4 d0 = *(const f32x4 *)(s_dt + u0), d1 = *(const f32x4 *)(s_dt + u0 + 4);
                const f32x4 c0 = *(const f32x4 *)(s_cs + u0), c1 = *(const f32x4 *)(s_cs + u0 + 4);
                const f32x4 e0 = *(const f32x4 *)(s_ce + u0), e1 = *(const f32x4 *)(s_ce + u0 + 4);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float cbv = (float)cb8[j];
                    const float dtu = j < 4 ? d0[j] : d1[j - 4];
                    const float csu = j < 4 ? c0[j] : c1[j - 4];
                    const float ceu = j < 4 ? e0[j] : e1[j - 4];
                    // the decay exponent of the right direction is the non-positive one
                    const float m = cbv * dtu * ex2(fminf(cs_t - csu, ceu - ce_t));
                    mf[j] = (_Float16)(16 * (kb & 1) + j == jd ? 2.f * cbv * dt_t + twoD : m);
                }
            } else {
                const f16x8 g8 = *(const f16x8 *)((U < tb ? s_gl : s_gu) + u0);
                mf = cb8 * (g8 * fac[U]);
            }
#pragma unroll
            for (int j = 0; j < YT; ++j) yacc[j] = mfma16(xa[pb0 + j - px0], mf, yacc[j]);
            // state update: Hf^T += (B^T w) x^T, the token weights applied along the contraction
            const f16x8 w8 = *(const f16x8 *)(s_w + u0);
            const f16x8 af = __builtin_bit_cast(f16x8, bfr[kb]);
#pragma unroll
            for (int i = 0; i < HT; ++i) hacc[i] = mfma16(af, xa[hpb0 + i - px0] * w8, hacc[i]);
        }

        // inter-chunk terms, one Y^T tile at a time: ef * (Hf C^T) + eb * (Hb C^T)
        const float ef = ex2(cs_t);
        const float eb = ex2(tot_c * LOG2E - ce_t);
#pragma unroll
        for (int j = 0; j < YT; ++j) {
            const int pb = pb0 + j;
            f32x16 yb = f32x16{};
#pragma unroll
            for (int kb = 0; kb < KS; ++kb)
                yb = mfma(frag_rm(hfl, SS, 32 * pb, 16 * kb), __builtin_bit_cast(bf16x8, cfr[kb]), yb);
#pragma unroll
            for (int e = 0; e < 16; ++e) yacc[j][e] += ef * yb[e];
            yb = f32x16{};
#pragma unroll
            for (int kb = 0; kb < KS; ++kb)
                yb = mfma(frag_rm(hbl, SS, 32 * pb, 16 * kb), __builtin_bit_cast(bf16x8, cfr[kb]), yb);
            // Y = acc + eb * yb into ybuf (lane: token t_tok, 4 consecutive p per group)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(yacc[j][4 * g4 + e] + eb * yb[4 * g4 + e]);
                *(bf16x4 *)&ybuf[t_tok * LY + 32 * pb + 8 * g4 + 4 * half] = v4;
            }
        }
        load_hinb();
        fetch_group(cn, 0);
        if (row_thread) {
            int pt = tid;
            pin(pt);
            s_rowy[pt & (NT - 1)] = rowc;
        }
        __syncthreads();  // ybuf complete; this chunk's other LDS reads are done

        // ---- store, then stage the next chunk ----
        store_y();
        if (c + 1 < c_hi) stage();
    }
}

// ---------------------------------------------------------------------------
// 5. Review tokens of x from the run sums of the fused state sweep: the mean over each pool block (its
// runs of 8 tokens along the run axis, every token of the block once), rx[b][j][c] with j in RMS order of
// the pooled grid. grid (ceil(C / 2048), R, batch); 8 channels per thread. axis: 0 t, 1 h, 2 w.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pool_runs(const __bf16 *__restrict__ xpart, bf16_t *__restrict__ rx,
                                                   int64_t C, uint32_t Tn, uint32_t Hn, uint32_t Wn, int pt, int ph,
                                                   int pw, int order, int axis)
{
    const int64_t ch = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (ch >= C) return;
    const uint32_t j = blockIdx.y, b = blockIdx.z, R = gridDim.y;
    const uint32_t Tp = Tn / pt, Hp = Hn / ph, Wp = Wn / pw;
    const uint32_t np = rms_index32(j, order, Tp, Hp, Wp);
    const uint32_t tq = np / (Hp * Wp), hq = (np / Wp) % Hp, wq = np % Wp;
    const size_t nrun = (size_t)Tn * Hn * Wn / 8;
    const int st = axis == 0 ? 8 : 1, sh = axis == 1 ? 8 : 1, sw = axis == 2 ? 8 : 1;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int dt_ = 0; dt_ < pt; dt_ += st)
        for (int dh = 0; dh < ph; dh += sh)
            for (int dw = 0; dw < pw; dw += sw) {
                const uint32_t t = tq * pt + dt_, h = hq * ph + dh, w = wq * pw + dw;
                const size_t run = axis == 2 ? ((size_t)t * Hn + h) * (Wn / 8) + w / 8
                                 : axis == 1 ? ((size_t)t * (Hn / 8) + h / 8) * Wn + w
                                             : ((size_t)(t / 8) * Hn + h) * Wn + w;
                const u32x4 v = __builtin_nontemporal_load((const u32x4 *)(xpart + ((size_t)b * nrun + run) * C + ch));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += lo_f(v[e]);
                    acc[2 * e + 1] += hi_f(v[e]);
                }
            }
    const float inv = 1.f / (float)(pt * ph * pw);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    *(u32x4 *)(rx + ((size_t)b * R + j) * C + ch) = o;
}

// The fused review pooling applies when every aligned group of 8 consecutive positions of the scan lies in
// one pool block: the scan's fastest axis (w for orders 0 and 4, h for order 1, t for orders 2 and 3) has a
// pool extent that is a multiple of 8 (so the grid's extent along it is too) and x rows are 64 channels.
// Returns that axis (0 t, 1 h, 2 w), or -1.
int fused_pool_axis(const SsdProblem &p)
{
    if (p.R <= 0 || p.chunk != 128) return -1;
    const int axis = (p.order == 0 || p.order == 4) ? 2 : p.order == 1 ? 1 : 0;
    const int pool = axis == 2 ? p.pool_w : axis == 1 ? p.pool_h : p.pool_t;
    return pool % 8 == 0 ? axis : -1;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Plan {
    int nseg, segch, nsegT;
    size_t perm, dtT, csT, cb, cfrag, bfrag, hbl, delta, segF, segB, segA, hinF, hinB, ytrash, rx, rB, rdt, rdtT, rcsT,
        xpart, total;
};

Plan make_plan(const SsdProblem &p)
{
    Plan pl{};
    const size_t B = p.batch, Hs = p.nheads, S = p.d_state, Q = p.chunk, PS = (size_t)P * S;
    const size_t Lpad = (size_t)p.nch * Q;
    // About five rounds of the output sweep's resident workgroups (two per CU) over the whole launch.
    int want = (int)((2560 + B * Hs - 1) / (B * Hs));
    if (want < 1) want = 1;
    if (want > p.nch) want = p.nch;
    pl.segch = (p.nch + want - 1) / want;
    pl.nseg = (p.nch + pl.segch - 1) / pl.segch;
    pl.nsegT = pl.nseg + (p.R > 0 ? 1 : 0);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    pl.perm = take((size_t)p.N * 4);
    pl.dtT = take(B * Hs * Lpad * 4);
    pl.csT = take(B * Hs * Lpad * 4);
    pl.cb = take(B * p.ngroups * p.nch * Q * Q * 2);
    pl.cfrag = take(B * p.ngroups * p.nch * Q * S * 2);
    pl.bfrag = take(B * p.ngroups * p.nch * Q * S * 2);
    pl.hbl = take(B * Hs * p.nch * PS * 2);
    pl.delta = take(B * Hs * p.nch * 4);
    pl.segF = take(B * Hs * pl.nsegT * PS * 4);
    pl.segB = take(B * Hs * pl.nsegT * PS * 4);
    pl.segA = take(B * Hs * pl.nsegT * 4);
    pl.hinF = take(B * Hs * pl.nseg * PS * 4);
    pl.hinB = take(B * Hs * pl.nseg * PS * 2);
    pl.ytrash = take((size_t)P * 2);
    if (p.R > 0) {
        const size_t Rpad = (size_t)p.nchR * Q;
        pl.rx = take(B * p.R * Hs * P * 2);
        pl.rB = take(B * p.R * p.ngroups * S * 2);
        pl.rdt = take(B * p.R * Hs * 4);
        pl.rdtT = take(B * Hs * Rpad * 4);
        pl.rcsT = take(B * Hs * Rpad * 4);
        // run sums of the fused pooling (any order may take it: sized for all)
        SsdProblem q = p;
        bool any = false;
        for (int o = 0; o <= 4 && !any; ++o) {
            q.order = o;
            any = fused_pool_axis(q) >= 0;
        }
        if (any) pl.xpart = take(B * (size_t)(p.N / 8) * Hs * P * 2);
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
    uint32_t *perm = (uint32_t *)(w + pl.perm);
    float *dtT = (float *)(w + pl.dtT), *csT = (float *)(w + pl.csT);
    _Float16 *cb = (_Float16 *)(w + pl.cb);
    __bf16 *cfrag = (__bf16 *)(w + pl.cfrag);
    _Float16 *bfrag = (_Float16 *)(w + pl.bfrag);
    __bf16 *hbl = (__bf16 *)(w + pl.hbl);
    float *delta = (float *)(w + pl.delta), *segF = (float *)(w + pl.segF), *segB = (float *)(w + pl.segB);
    float *segA = (float *)(w + pl.segA), *hinF = (float *)(w + pl.hinF);
    __bf16 *hinB = (__bf16 *)(w + pl.hinB);
    const int Hs = p.nheads, G = p.ngroups, Bn = (int)p.batch;
    const uint32_t N = (uint32_t)p.N, Lpad = (uint32_t)(p.nch * Q);
    const uint32_t T = (uint32_t)p.T, H = (uint32_t)p.H, W = (uint32_t)p.W;
    const __bf16 *x = (const __bf16 *)a.x, *Bm = (const __bf16 *)a.b, *Cm = (const __bf16 *)a.c;

    const int pool_axis = fused_pool_axis(p);
    __bf16 *xpart = pool_axis >= 0 ? (__bf16 *)(w + pl.xpart) : nullptr;
    const uint32_t run_stride = pool_axis == 2 ? 1u : pool_axis == 1 ? W : H * W;
    {
        timing::Scope ts_(K_SSD_PREP, st);
        k_perm<<<(N + 255) / 256, 256, 0, st>>>(perm, N, p.order, T, H, W);
    }
    {
        timing::Scope ts_(K_SSD_PREP, st);
        ssd::prep_dt<true>(a.dt, a.a, dtT, csT, Hs, N, Lpad, Q, p.order, T, H, W, p.nch, Bn, st, perm);
    }
    {
        timing::Scope ts_(K_SSD_CB, st);
        k_cb<S, Q><<<dim3(p.nch, G, Bn), NT, 0, st>>>(Bm, Cm, perm, cb, cfrag, bfrag, G, N);
    }
    const uint64_t items = (uint64_t)Bn * pl.nseg * Hs;
    {
        timing::Scope ts_(K_SSD_STATES, st);
        if constexpr (Q == 128) {
            if (xpart) {
                k_states<S, Q, true><<<grid_of(items), NT, 0, st>>>(
                    x, bfrag, perm, dtT, csT, a.a, hbl, delta, segF, segB, segA, xpart, run_stride, N / 8, Hs, G, N,
                    Lpad, p.nch, pl.segch, pl.nseg, pl.nsegT, (uint32_t)items);
            }
        }
        if (!xpart)
            k_states<S, Q, false><<<grid_of(items), NT, 0, st>>>(x, bfrag, perm, dtT, csT, a.a, hbl, delta, segF, segB,
                                                                 segA, nullptr, 1u, 0u, Hs, G, N, Lpad, p.nch,
                                                                 pl.segch, pl.nseg, pl.nsegT, (uint32_t)items);
    }
    // Review tokens (after the main sweep, which leaves the run sums of x when the pooling is fused):
    // pooled x, B and dt, their dt table, and the review segment's summaries.
    if (p.R > 0) {
        bf16_t *rx = (bf16_t *)(w + pl.rx), *rB = (bf16_t *)(w + pl.rB);
        float *rdt = (float *)(w + pl.rdt), *rdtT = (float *)(w + pl.rdtT), *rcsT = (float *)(w + pl.rcsT);
        const uint32_t R = (uint32_t)p.R, Rpad = (uint32_t)(p.nchR * Q);
        const int64_t Cx = (int64_t)Hs * P, Cb = (int64_t)G * S;
        {
            timing::Scope ts_(K_SSD_POOL, st);
            if (xpart)
                k_pool_runs<<<dim3((Cx / 8 + 255) / 256, R, Bn), 256, 0, st>>>(
                    xpart, rx, Cx, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order, pool_axis);
            else
                ssd::k_pool8<bf16_t><<<dim3((Cx + 2047) / 2048, R, Bn), 256, 0, st>>>(
                    (const bf16_t *)a.x, rx, Cx, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        }
        {
            timing::Scope ts_(K_SSD_POOL, st);
            ssd::k_pool8<bf16_t><<<dim3((Cb + 2047) / 2048, R, Bn), 256, 0, st>>>(
                (const bf16_t *)a.b, rB, Cb, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        }
        {
            timing::Scope ts_(K_SSD_POOL, st);
            if (ssd::pool_f32x4_ok(a.dt, Hs))
                ssd::k_pool_f32x4<<<dim3(R, Bn), ssd::kPoolF4Threads, 0, st>>>(a.dt, rdt, Hs, T, H, W, p.pool_t, p.pool_h, p.pool_w,
                                                              p.order);
            else
                ssd::k_pool<float, float><<<dim3((Hs + 255) / 256, R, Bn), 256, 0, st>>>(
                    a.dt, rdt, Hs, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        }
        {
            timing::Scope ts_(K_SSD_PREP, st);
            ssd::prep_dt<false>(rdt, a.a, rdtT, rcsT, Hs, R, Rpad, Q, 0, 1, 1, R, p.nchR, Bn, st);
        }
        const uint64_t ritems = (uint64_t)Bn * Hs;
        {
            timing::Scope ts_(K_SSD_STATES, st);
            k_states_review<S, Q><<<grid_of(ritems), Q * 4, 0, st>>>((const __bf16 *)rx, (const __bf16 *)rB, rdtT, rcsT,
                                                                  a.a, segF, segB, segA, Hs, G, R, Rpad, p.nchR,
                                                                  p.nchR, 1, pl.nseg, pl.nsegT, (uint32_t)ritems);
        }
    }
    {
        timing::Scope ts_(K_SSD_SEG_PASS, st);
        k_seg_pass<<<dim3((P * S + 255) / 256, Hs, Bn), 256, 0, st>>>(segF, segB, segA, hinF, hinB, P * S, pl.nseg,
                                                                      pl.nsegT, p.R > 0 ? 1 : 0);
    }
    {
        timing::Scope ts_(K_SSD_OUT, st);
        k_out<S, Q><<<grid_of(items), NT, 0, st>>>(x, bfrag, cfrag, cb, perm, dtT, csT, a.a, a.d, hbl, delta, hinF,
                                                   hinB, (__bf16 *)a.y, (__bf16 *)(w + pl.ytrash), Hs, G, N, Lpad,
                                                   p.nch, pl.segch, pl.nseg, (uint32_t)items);
    }
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
