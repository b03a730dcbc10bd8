// Bidirectional Mamba2 scan on bf16 MFMA (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Same chunked (state space duality) evaluation as the portable path, with
// the chunk states kept on chip. The sequence of each head is cut into
// segments of whole chunks; a workgroup of Q/16 waves (two per SIMD at
// Q = 128) owns one (head, segment):
//
//  1. states   sweeps its segment right to left, carrying the backward state
//              G in MFMA accumulators. Before adding chunk c it stores G (the
//              backward state entering c from the right, from zero at the
//              segment end) as bf16; it also accumulates the segment's forward
//              end state F. Ends with the segment summaries G, F and sum(dt A).
//              The review tokens form one extra segment whose G and F are the
//              initial states of the two directions.
//  2. seg pass turns summaries into the true states at every segment border.
//  3. cb       C_t . B_u (fp16) for every chunk (shared by all heads of a group).
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
// Data layout on chip: x and B chunks are staged in LDS in their natural
// row-major layout (token rows) with plain 16-byte copies; the operands of the
// contractions over tokens are read with the gfx950 LDS transpose read
// (ds_read_b64_tr_b16), which hands each lane 4 consecutive rows of one
// column. C rows, CB rows and the stored states are contiguous along their
// contraction axis and are used as MFMA fragments directly.
//
// Decay weights of M: inside the 32x32 diagonal block of a lane's token block
// each weight is one exp2; in the blocks below (above) it, exp(cs_t - cs_u)
// (exp(ce_u - ce_t)) is split at the block edge into a per-lane factor and a
// per-token factor, both <= 1, so no exponent is evaluated per element.
//
// Scan order: a table of the RMS permutation (scan position -> canonical
// token) is built once per call; every gather reads it instead of dividing.
// Block ids are remapped so that the workgroups resident on one XCD work on
// consecutive heads of one segment and share B, C and CB in that XCD's L2.
#include "common.hpp"
#include "launch.hpp"
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

// MFMA operand fragment from a row-major [k][n] LDS tile (row stride ld):
// lane l gets column n_base + l % 32 at rows k_base + 8 (l / 32) + 0..7.
__device__ __forceinline__ bf16x8 frag_tr(const __bf16 *tile, int ld, int k_base, int n_base)
{
    const int l = threadIdx.x & 63, g = l >> 4, s = l & 15;
    const __bf16 *p = tile + (k_base + 8 * (g >> 1) + (s >> 2)) * ld + n_base + 16 * (g & 1) + 4 * (s & 3);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * ld));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// MFMA operand fragment from a row-major [m][k] LDS tile: lane l gets row
// m_base + l % 32 at columns k_base + 8 (l / 32) + 0..7.
__device__ __forceinline__ bf16x8 frag_rm(const __bf16 *tile, int ld, int m_base, int k_base)
{
    const int l = threadIdx.x & 63;
    return *(const bf16x8 *)(tile + (m_base + (l & 31)) * ld + k_base + 8 * (l >> 5));
}

// Q token rows of COLS bf16 each, split in 16-byte units over the workgroup.
// Row u of the chunk is read from global row srow[u] (an LDS table of the
// chunk's rows; ~0u marks a position past the end). Loads are unconditional:
// a position past the end reads row 0 of the batch, a finite row that the
// kernels multiply by that position's weight dt = 0 (or never store), so no
// select waits on the load.
template <int Q, int COLS, int NT>
struct Rows {
    static constexpr int UPR = COLS / 8;
    static constexpr int PER = Q * UPR / NT;
    static_assert(Q * UPR % NT == 0, "tile must split evenly over the workgroup");
    u32x4 r[PER];

    __device__ __forceinline__ static int row_of(int it) { return (threadIdx.x + NT * it) / UPR; }
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

// CB of a chunk is stored in 8-element pieces in the order the output sweep reads them: thread lane l
// of wave w (Q/16 waves) owns row t = 16 w + l % 16 and, in every 32-column block U, columns
// 32 U + 8 (l / 16) + 0..7. Returns the element offset of piece (t, U, m = (u % 32) / 8).
template <int Q>
__device__ __forceinline__ int cb_piece(int t, int U, int m)
{
    return (((U * (Q / 16) + (t >> 4)) * 64) + (t & 15) + 16 * m) * 8;
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
// 1. Right-to-left segment sweep: stored backward chunk states + summaries.
// grid = 8 * ceil(batch * nseg * nheads / 8); item = (b * nseg + seg) * nheads + h.
// MAIN: the main sequence (x rows through perm, B from the fp16 scan-order copy; stores the per-chunk
// states); else the review sequence (rows in order, B pooled bf16; summaries only).
// Each wave owns (s-block, p-block) tile pairs: the backward state G^T and the forward sum F^T of the
// same tile share both operand tiles, B^T and x (fp16); the per-token weights of the two sums,
// dt exp(ce) and dt exp(tot - cs + logD), are applied to the x operand in registers (packed fp16).
// The x rows and per-token values of the chunk two to the left (and B of the next one) are loaded every
// step (clamped at the segment start), and the per-step stores are made by every wave, so the
// compiler's memory waits are not widened by paths that skip them.
// ---------------------------------------------------------------------------
template <int S, int Q, bool MAIN>
__global__ __launch_bounds__(Q * 4) void k_states(const __bf16 *__restrict__ x, const __bf16 *__restrict__ Bm,
                                                  const _Float16 *__restrict__ b16,
                                                  const uint32_t *__restrict__ perm, const float *__restrict__ dtT,
                                                  const float *__restrict__ csT, const float *__restrict__ A,
                                                  __bf16 *__restrict__ hb_local, float *__restrict__ delta,
                                                  float *__restrict__ segF, float *__restrict__ segB,
                                                  float *__restrict__ segA, int nheads, int G, uint32_t L,
                                                  uint32_t Lpad, int nch, int segch, int nseg, int seg_base,
                                                  int nseg_total, uint32_t total_items)
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
    const size_t gch = ((size_t)b * G + g) * nch;
    // x rows and per-token values are fetched two chunks ahead into two alternating
    // register stages (their HBM latency exceeds a chunk's work). B of the main pass
    // (contiguous fp16 rows of group data, L2-resident) comes one chunk ahead; the
    // review pass gathers B with the chunk's row table, so it rides in the stage.
    struct Stage {
        Rows<Q, P, NT> xr;
        u32x4 bq[BPER];  // review pass: B pieces k = tid + NT it (row k / (S / 8), 8 columns at 8 (k % (S / 8)))
        float tok_d, tok_c, tot;
    };
    Stage stA, stB;
    u32x4 bm[BPER];       // main pass: B of the chunk after the current one, same pieces
    uint32_t pnext = 0u;  // row-table entry of the chunk after the one fetched last
    bool pvalid = false;
    auto fetch = [&](Stage &stg, int c) {
        // The row-table load first: the compiler may move its use above the next barrier, and a wait for
        // it then covers only older loads.
        const int tq = tid & (Q - 1);
        const uint32_t i = (uint32_t)(c - 1) * Q + tq;
        pvalid = c > c_lo && i < L;
        if constexpr (MAIN)
            pnext = perm[pvalid ? i : 0u];  // selected against pvalid where it is stored
        else
            pnext = i;
        stg.xr.load(x + (size_t)h * P, (size_t)nheads * P, s_row, (size_t)b * L);
        if constexpr (!MAIN) {
            Rows<Q, S, NT> br;
            br.load(Bm + (size_t)g * S, (size_t)G * S, s_row, (size_t)b * L);
#pragma unroll
            for (int it = 0; it < BPER; ++it) stg.bq[it] = br.r[it];
        }
        const size_t crow0 = drow + (size_t)c * Q;
        stg.tok_d = dtT[crow0 + tq];
        stg.tok_c = csT[crow0 + tq];
        stg.tot = csT[crow0 + Q - 1];
    };
    auto fetch_b = [&](int c) {
        if constexpr (MAIN) {
            const _Float16 *src = b16 + (gch + c) * (size_t)(Q * S);
#pragma unroll
            for (int it = 0; it < BPER; ++it) bm[it] = *(const u32x4 *)(src + 8 * (tid + NT * it));
        }
    };
    // Prologue: rows and data of the rightmost chunk, then the rows and x of the one before.
    if (row_thread) s_row[tid] = seq_row(MAIN ? perm : nullptr, (uint32_t)(c_hi - 1) * Q + tid, L);
    __syncthreads();
    fetch(stA, c_hi - 1);
    fetch_b(c_hi - 1);
    __syncthreads();  // every lane has read the rows of chunk c_hi - 1
    s_row[tid & (Q - 1)] = pvalid ? pnext : ~0u;
    __syncthreads();
    fetch(stB, max(c_hi - 2, c_lo));  // a one-chunk segment: issued, unused
    float logD = 0.f;  // sum of dt*A over the chunks right of the current one

    auto step = [&](Stage &cur, int c) {
        if constexpr (MAIN) {
            // Backward state entering chunk c from the right, in accumulator order (see hb_piece).
            if (active) {
                __bf16 *dst = hb_local + (bh * nch + c) * (size_t)(P * S);
#pragma unroll
                for (int i = 0; i < TP; ++i) {
                    const int j = wave * TP + i;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        bf16x8 v8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) v8[e] = (__bf16)accG[i][8 * q + e];
                        *(bf16x8 *)(dst + ((j * 2 + q) * 64 + lane) * 8) = v8;
                    }
                }
            }
            delta[bh * nch + c] = ex2(logD * LOG2E);  // every thread writes the same value
        }

        __syncthreads();  // previous chunk's MFMA reads of LDS and the row-table reads are done
        // The staged values are used from here on (their loads had two steps to complete).
#pragma unroll
        for (int it = 0; it < Rows<Q, P, NT>::PER; ++it) pin(cur.xr.r[it]);
#pragma unroll
        for (int it = 0; it < BPER; ++it) {
            if constexpr (MAIN)
                pin(bm[it]);
            else
                pin(cur.bq[it]);
        }
        pin(cur.tok_d);
        pin(cur.tok_c);
        pin(cur.tot);
        pin(pnext);
        const float tot_c = cur.tot;
        cur.xr.template store_f16<LX>((__bf16 *)xn);
#pragma unroll
        for (int it = 0; it < BPER; ++it) {
            const int k = tid + NT * it;
            u32x4 v;
            if constexpr (MAIN) {
                v = bm[it];
            } else {
                v = cur.bq[it];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = pack2h(lo_f(v[e]), hi_f(v[e]));
            }
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

        // B (needed next step) before x (needed in two): waits complete in issue order.
        fetch_b(max(c - 1, c_lo));
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
    float run = has_review ? F[(size_t)nseg * PS] : 0.f;
    for (int j = 0; j < nseg; ++j) {
        hinF[(bh * nseg + j) * PS + e] = run;
        run = ex2(sa[j] * LOG2E) * run + F[(size_t)j * PS];
    }
    run = has_review ? Bk[(size_t)nseg * PS] : 0.f;
    for (int j = nseg - 1; j >= 0; --j) {
        hinB[(bh * nseg + j) * PS + e] = (__bf16)run;
        run = ex2(sa[j] * LOG2E) * run + Bk[(size_t)j * PS];
    }
}

// ---------------------------------------------------------------------------
// 3. Per chunk and group (grid (nch, G, batch)), for the output sweep:
//    cb    CB[t][u] = C_t . B_u (fp16), computed as CB^T = B C^T so each lane holds 4 consecutive u of one t,
//          stored in the output sweep's piece order (cb_piece);
//    b16   the chunk's B rows in scan order, as fp16 ([Q][S]);
//    cfrag the chunk's C rows in MFMA operand order: for token block tb and k-block kb, lane l's 8 values
//          C[32 tb + l % 32][16 kb + 8 (l / 32) + 0..7] are the l-th 16 bytes of a 1 KB block, so the sweep
//          reads each operand with one contiguous load per wave.
// ---------------------------------------------------------------------------
template <int S, int Q>
__global__ __launch_bounds__(NT) void k_cb(const __bf16 *__restrict__ Bm, const __bf16 *__restrict__ Cm,
                                           const uint32_t *__restrict__ perm, _Float16 *__restrict__ cb,
                                           _Float16 *__restrict__ b16, __bf16 *__restrict__ cfrag, int G, uint32_t L)
{
    const uint32_t c = blockIdx.x;
    const int g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int TB = Q / 32;
    constexpr int TILES = TB * TB / 4;  // per wave
    const size_t rs = (size_t)G * S;
    const size_t chunk = ((size_t)b * G + g) * gridDim.x + c;
    _Float16 *out = cb + chunk * (size_t)(Q * Q);
#pragma unroll
    for (int k = 0; k < TILES; ++k) {
        const int ti = wave + 4 * k;
        const int ub = ti / TB, tb = ti % TB;
        const uint32_t iu = c * Q + 32 * ub + col, itk = c * Q + 32 * tb + col;
        const bool uok = iu < L, tok = itk < L;
        const __bf16 *brow = Bm + ((size_t)b * L + (uok ? perm[iu] : 0u)) * rs + (size_t)g * S;
        const __bf16 *crow = Cm + ((size_t)b * L + (tok ? perm[itk] : 0u)) * rs + (size_t)g * S;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kb = 0; kb < S / 16; ++kb) {
            u32x4 av = *(const u32x4 *)(brow + 16 * kb + 8 * half);
            u32x4 bv = *(const u32x4 *)(crow + 16 * kb + 8 * half);
            av = uok ? av : u32x4{0, 0, 0, 0};
            bv = tok ? bv : u32x4{0, 0, 0, 0};
            acc = mfma(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc);
        }
        // acc: rows u = 32ub + 8g4 + 4half + j, column t = 32tb + col; stored in piece order (see cb_piece)
        const int t = 32 * tb + col;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            f16x4 v4;
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] = (_Float16)acc[4 * g4 + j];
            *(f16x4 *)(out + cb_piece<Q>(t, ub, g4) + 4 * half) = v4;
        }
    }
    // B rows as fp16 (exact for bf16 values in fp16's normal range) and C rows in operand order.
    constexpr int PIECES = Q * S / 8, PER = PIECES / NT;
    static_assert(PIECES % NT == 0, "pieces must split evenly");
    _Float16 *bo = b16 + chunk * (size_t)(Q * S);
    __bf16 *co = cfrag + chunk * (size_t)(Q * S);
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int k = tid + NT * it;
        {
            const int row = k / (S / 8), c8 = k % (S / 8);
            const uint32_t i = c * Q + row;
            const u32x4 v = *(const u32x4 *)(Bm + ((size_t)b * L + (i < L ? perm[i] : 0u)) * rs + (size_t)g * S + 8 * c8);
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = i < L ? pack2h(lo_f(v[e]), hi_f(v[e])) : 0u;
            *(u32x4 *)(bo + (size_t)row * S + 8 * c8) = o;
        }
        {
            const int l = k % 64, kb = (k / 64) % (S / 16), tb = k / (64 * (S / 16));
            const uint32_t i = c * Q + 32 * tb + (l & 31);
            const u32x4 v = *(const u32x4 *)(Cm + ((size_t)b * L + (i < L ? perm[i] : 0u)) * rs + (size_t)g * S +
                                              16 * kb + 8 * (l >> 5));
            *(u32x4 *)(co + 8 * (size_t)k) = i < L ? v : u32x4{0, 0, 0, 0};
        }
    }
}

// ---------------------------------------------------------------------------
// 4. Left-to-right output sweep. Same grid/items as k_states (main segments).
//
// Per chunk, three phases separated by barriers:
//   build  this chunk's C operands are requested (contiguous, in operand order), then the next chunk's
//          data; Hf advances on fp16 MFMA (Hf^T += B^T (w x)^T with w = dt exp(tot - cs) applied to the
//          x operand in registers); every thread turns one 8-column piece of CB per 32-column block into M
//          in place (fp16, row t = token); the 16 rows of a wave lie in one 32-row block, so each piece is
//          uniformly below, on or above the diagonal block across the wave;
//   use    Y^T = X^T M^T + ef (Hf C^T) + eb (Hb C^T); Y goes to LDS as bf16 rows;
//   store  Y rows leave as contiguous 16-byte pieces; the next chunk is staged: x (fp16), B (fp16), the
//          forward state Hf (from the accumulators), the backward state Hb = stored local state + decay *
//          border state, CB, and the per-token decay data.
// Every load and store in the loop is unconditional (a lane past the end of the sequence reads row 0
// and stores into a scratch row), and no load result crosses the loop edge, so the compiler's memory
// waits stay exact.
// ---------------------------------------------------------------------------
template <int S, int Q>
__global__ __launch_bounds__(Q * 4) void k_out(const __bf16 *__restrict__ x, const _Float16 *__restrict__ b16,
                                            const __bf16 *__restrict__ cfrag, const _Float16 *__restrict__ cb,
                                            const uint32_t *__restrict__ perm,
                                            const float *__restrict__ dtT, const float *__restrict__ csT,
                                            const float *__restrict__ A, const float *__restrict__ Dv,
                                            const __bf16 *__restrict__ hb_local, const float *__restrict__ delta,
                                            const float *__restrict__ hinF, const __bf16 *__restrict__ hinB,
                                            __bf16 *__restrict__ y, __bf16 *__restrict__ ytrash, int nheads, int G,
                                            uint32_t N, uint32_t Lpad, int nch, int segch, int nseg,
                                            uint32_t total_items)
{
    constexpr int NT = Q * 4, NW = Q / 16;  // Q/16 waves, two per SIMD at Q = 128
    constexpr int LX = P + XPAD, LB = S + XPAD, SS = S + 8, LM = Q + 8, LY = P + 8;
    constexpr int UB = Q / 32;              // 32-column blocks of M
    __shared__ _Float16 xn[Q * LX];  // x as fp16: operand of the intra-chunk product and of the state update
    __shared__ _Float16 bn[Q * LB];  // B as fp16
    __shared__ __bf16 hfl[P * SS];   // forward state entering the chunk, [p][s]
    __shared__ __bf16 hbl[P * SS];   // backward state entering the chunk from the right, [p][s]
    __shared__ __attribute__((aligned(16))) _Float16 mt[Q * LM];  // CB, then M[t][u] (fp16)
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
    const bool row_thread = wave < Q / 64;  // tid < Q
    // One Y^T tile per wave: t-block wave / 2, p-block wave % 2.
    const int tb = wave >> 1, pb = wave & 1;
    // Role in building M: row mrow, columns 32 U + 8 msub + 0..7 for every block U (one row per lane of
    // each 16-lane group, so LDS accesses of a group hit distinct banks); the wave's rows
    // 16 wave .. 16 wave + 15 all lie in row block wave / 2.
    const int mrow = 16 * wave + (lane & 15), msub = lane >> 4, mtb = wave >> 1;
    // Hf^T tiles (S/32 s-blocks x 2 p-blocks) over the waves: HT per wave, or one
    // tile for the first S/16 waves when there are fewer tiles than waves.
    constexpr int HTILES = S / 16;
    constexpr int HT = HTILES >= NW ? HTILES / NW : 1;
    const bool hact = wave < HTILES;
    const int hsb = (wave * HT) >> 1;
    const int hpb0 = (wave * HT) & 1;
    const float a = A[h];
    const float twoD = 2.f * Dv[h];
    constexpr int PS = P * S;

    f32x16 hacc[HT];
#pragma unroll
    for (int i = 0; i < HT; ++i) hacc[i] = f32x16{};
    if (hact) {
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
    // Border state of the backward direction (bf16), for this thread's staging chunks.
    constexpr int HBC = PS / 8 / NT;  // 16-byte chunks of Hb per thread
    // (pieces in the stored states' accumulator order; see hb_piece)
    u32x4 hinb[HBC];
    {
        const __bf16 *src = hinB + (bh * nseg + seg) * (size_t)PS;
#pragma unroll
        for (int it = 0; it < HBC; ++it) {
            const HbPiece pc = hb_piece(tid + NT * it);
            const u32x2 lo = *(const u32x2 *)(src + pc.p * S + pc.s_a);
            const u32x2 hi = *(const u32x2 *)(src + pc.p * S + pc.s_a + 8);
            hinb[it] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    }

    Rows<Q, P, NT> xr;
    constexpr int BPER = Q * S / 8 / NT;  // 16-byte pieces of the B tile per thread
    const size_t gch = ((size_t)b * G + g) * nch;  // chunk index base of this group
    const int t_tok = 32 * tb + col;  // this lane's token inside the chunk (Y^T column)

    // Staging data of the next chunk: loaded in the build phase, consumed by the staging at the end of
    // the same iteration.
    u32x4 bru[BPER];
    u32x4 hbr[HBC];
    u32x4 cbr[UB];  // CB row pieces, for mt
    float tok_d = 0.f, tok_c = 0.f, tot = 0.f, dl = 0.f;
    uint32_t pnext = 0u;
    bool pvalid = false;
    // The next chunk's data comes in two groups: per-head data that misses to HBM (x, the stored
    // states, per-token values) early in the build phase, and the chunk's group data that other
    // heads have just read (B, CB; L2-resident) in the use phase, where it overlaps the MFMAs
    // instead of queueing in one burst before them.
    auto fetch = [&](int c) {
        xr.load(x + (size_t)h * P, (size_t)nheads * P, s_row, (size_t)b * N);
        const __bf16 *src = hb_local + (bh * nch + c) * (size_t)PS;
#pragma unroll
        for (int it = 0; it < HBC; ++it) hbr[it] = *(const u32x4 *)(src + 8 * (tid + NT * it));
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
    auto fetch_group = [&](int c) {
        const _Float16 *bsrc = b16 + (gch + c) * (size_t)(Q * S);
#pragma unroll
        for (int it = 0; it < BPER; ++it) bru[it] = *(const u32x4 *)(bsrc + 8 * (tid + NT * it));
        const _Float16 *cbs = cb + (gch + c) * (size_t)(Q * Q) + 8 * (size_t)tid;  // cb_piece(mrow, U, msub)
#pragma unroll
        for (int U = 0; U < UB; ++U) cbr[U] = *(const u32x4 *)(cbs + U * (Q / 16) * 512);
    };
    uint32_t rowc = 0u;  // row-thread: global row of token tid of the staged chunk (~0u past the end)
    auto stage = [&]() {
        xr.template store_f16<LX>((__bf16 *)xn);
#pragma unroll
        for (int it = 0; it < BPER; ++it) {
            const int k = tid + NT * it;
            *(u32x4 *)&bn[(k / (S / 8)) * LB + 8 * (k % (S / 8))] = bru[it];
        }
        if (hact) {
#pragma unroll
            for (int i = 0; i < HT; ++i)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    bf16x4 v4;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v4[j] = (__bf16)hacc[i][4 * g4 + j];
                    *(bf16x4 *)&hfl[(32 * (hpb0 + i) + col) * SS + 32 * hsb + 8 * g4 + 4 * half] = v4;
                }
        }
#pragma unroll
        for (int it = 0; it < HBC; ++it) {
            const HbPiece pc = hb_piece(tid + NT * it);
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack2(lo_f(hbr[it][e]) + dl * lo_f(hinb[it][e]), hi_f(hbr[it][e]) + dl * hi_f(hinb[it][e]));
            *(u32x2 *)&hbl[pc.p * SS + pc.s_a] = u32x2{o[0], o[1]};
            *(u32x2 *)&hbl[pc.p * SS + pc.s_a + 8] = u32x2{o[2], o[3]};
        }
#pragma unroll
        for (int U = 0; U < UB; ++U) *(u32x4 *)(mt + mrow * LM + 32 * U + 8 * msub) = cbr[U];
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
            s_dt[tid] = tok_d;
            s_cs[tid] = cs2;
            s_ce[tid] = ce2;
            // below-diagonal blocks: exp(cs_end - cs_u); above: exp(ce_u - ce_start); both <= 1
            s_gl[tid] = (_Float16)(tok_d * ex2(blk_cs_end * LOG2E - cs2));
            s_gu[tid] = (_Float16)(tok_d * ex2(ce2 - (blk_cs0 - blk_dt0 * a) * LOG2E));
            // weight of token u in the state carried out of the chunk
            s_w[tid] = (_Float16)(tok_d * ex2(tot * LOG2E - cs2));
            rowc = s_row[tid];
            s_row[tid] = pvalid ? pnext : ~0u;
        }
    };
    // Output rows of the chunk in ybuf: contiguous 16-byte pieces (a past-the-end row goes to scratch).
    auto store_y = [&]() {
#pragma unroll
        for (int it = 0; it < Q * (P / 8) / NT; ++it) {
            const int k = tid + NT * it;
            const int t = k / (P / 8), p8 = 8 * (k % (P / 8));
            const uint32_t r = s_rowy[t];
            __bf16 *dst = r != ~0u ? y + (((size_t)b * N + r) * nheads + h) * P + p8 : ytrash + p8;
            *(u32x4 *)dst = *(const u32x4 *)&ybuf[t * LY + p8];
        }
    };

    // Prologue: rows of the first chunk, its data, staged.
    if (row_thread) s_row[tid] = seq_row(perm, (uint32_t)c_lo * Q + tid, N);
    __syncthreads();
    fetch(c_lo);
    fetch_group(c_lo);
    __syncthreads();
    stage();

    for (int c = c_lo; c < c_hi; ++c) {
        __syncthreads();  // staged chunk c visible

        // ---- build ----
        const float tot_c = tot;
        const int cn = c + 1 < c_hi ? c + 1 : c;  // on the last iteration the loads are issued but unused
        u32x4 cfr[S / 16];  // C operands of this lane's token: contiguous 1 KB per wave and k-block
        {
            const __bf16 *src = cfrag + (gch + c) * (size_t)(Q * S) + (size_t)tb * (S / 16) * 512 + 8 * lane;
#pragma unroll
            for (int kb = 0; kb < S / 16; ++kb) cfr[kb] = *(const u32x4 *)(src + 512 * kb);
        }
        fetch(cn);

        // Hf = exp(tot) Hf + sum_u w_u x_u B_u^T (as Hf^T = B^T (w x)^T, fp16 operands)
        if (hact) {
            const float dec = ex2(tot_c * LOG2E);
#pragma unroll
            for (int i = 0; i < HT; ++i) hacc[i] *= dec;
#pragma unroll
            for (int kb = 0; kb < Q / 16; ++kb) {
                const f16x8 af = __builtin_bit_cast(f16x8, frag_tr((const __bf16 *)bn, LB, 16 * kb, 32 * hsb));
                const f16x8 w8 = *(const f16x8 *)(s_w + 16 * kb + 8 * half);
#pragma unroll
                for (int i = 0; i < HT; ++i) {
                    const f16x8 xv = __builtin_bit_cast(f16x8, frag_tr((const __bf16 *)xn, LX, 16 * kb, 32 * (hpb0 + i)));
                    hacc[i] = mfma16(af, xv * w8, hacc[i]);
                }
            }
        }

        {
            const float cs_t = s_cs[mrow], ce_t = s_ce[mrow], dt_t = s_dt[mrow];
            _Float16 *mrw = mt + mrow * LM + 8 * msub;
#pragma unroll
            for (int U = 0; U < UB; ++U) {
                const int u0 = 32 * U + 8 * msub;
                const f16x8 cb8 = *(const f16x8 *)(mrw + 32 * U);
                f16x8 mf;
                if (U == mtb) {
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
                        mf[j] = (_Float16)(u0 + j == mrow ? 2.f * cbv * dt_t + twoD : m);
                    }
                } else if (U < mtb) {
                    const f16x8 g8 = *(const f16x8 *)(s_gl + u0);
                    mf = cb8 * (g8 * (_Float16)ex2(cs_t - s_cs[32 * U + 31]));
                } else {
                    const f16x8 g8 = *(const f16x8 *)(s_gu + u0);
                    mf = cb8 * (g8 * (_Float16)ex2(s_ce[32 * U] - ce_t));
                }
                *(f16x8 *)(mrw + 32 * U) = mf;
            }
        }
        __syncthreads();  // M complete

        // ---- use ----
        fetch_group(cn);
        f32x16 yacc = f32x16{}, yb = f32x16{};
        // intra-chunk term X^T M^T (fp16 MFMA)
#pragma unroll
        for (int kb = 0; kb < Q / 16; ++kb)
            yacc = mfma16(__builtin_bit_cast(f16x8, frag_tr((const __bf16 *)xn, LX, 16 * kb, 32 * pb)),
                          *(const f16x8 *)(mt + t_tok * LM + 16 * kb + 8 * half), yacc);
        // forward inter-chunk term: ef * (Hf C^T)
#pragma unroll
        for (int kb = 0; kb < S / 16; ++kb)
            yb = mfma(frag_rm(hfl, SS, 32 * pb, 16 * kb), __builtin_bit_cast(bf16x8, cfr[kb]), yb);
        {
            const float ef = ex2(s_cs[t_tok]);
#pragma unroll
            for (int j = 0; j < 16; ++j) yacc[j] += ef * yb[j];
        }
        yb = f32x16{};
        // backward inter-chunk term: eb * (Hb C^T)
#pragma unroll
        for (int kb = 0; kb < S / 16; ++kb)
            yb = mfma(frag_rm(hbl, SS, 32 * pb, 16 * kb), __builtin_bit_cast(bf16x8, cfr[kb]), yb);
        const float eb = ex2(tot_c * LOG2E - s_ce[t_tok]);
        // Y = acc + eb * yb into ybuf (lane: token t_tok, 4 consecutive p per group)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 v4;
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] = (__bf16)(yacc[4 * g4 + j] + eb * yb[4 * g4 + j]);
            *(bf16x4 *)&ybuf[t_tok * LY + 32 * pb + 8 * g4 + 4 * half] = v4;
        }
        if (row_thread) s_rowy[tid] = rowc;
        __syncthreads();  // ybuf complete; this chunk's other LDS reads are done

        // ---- store, then stage the next chunk ----
        store_y();
        if (c + 1 < c_hi) stage();
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Plan {
    int nseg, segch, nsegT;
    size_t perm, dtT, csT, cb, b16, cfrag, hbl, delta, segF, segB, segA, hinF, hinB, ytrash, rx, rB, rdt, rdtT, rcsT,
        total;
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
    pl.perm = take((size_t)p.N * 4);
    pl.dtT = take(B * Hs * Lpad * 4);
    pl.csT = take(B * Hs * Lpad * 4);
    pl.cb = take(B * p.ngroups * p.nch * Q * Q * 2);
    pl.b16 = take(B * p.ngroups * p.nch * Q * S * 2);
    pl.cfrag = take(B * p.ngroups * p.nch * Q * S * 2);
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
    }
    pl.total = off;
    return pl;
}

unsigned grid_of(uint64_t items) { return (unsigned)((items + 7) / 8 * 8); }

template <int S, int Q>
hipError_t run(const SsdProblem &p, const SsdArgs &a, void *ws, hipStream_t st, hipEvent_t before_out)
{
    const Plan pl = make_plan(p);
    char *w = (char *)ws;
    uint32_t *perm = (uint32_t *)(w + pl.perm);
    float *dtT = (float *)(w + pl.dtT), *csT = (float *)(w + pl.csT);
    _Float16 *cb = (_Float16 *)(w + pl.cb), *b16 = (_Float16 *)(w + pl.b16);
    __bf16 *cfrag = (__bf16 *)(w + pl.cfrag);
    __bf16 *hbl = (__bf16 *)(w + pl.hbl);
    float *delta = (float *)(w + pl.delta), *segF = (float *)(w + pl.segF), *segB = (float *)(w + pl.segB);
    float *segA = (float *)(w + pl.segA), *hinF = (float *)(w + pl.hinF);
    __bf16 *hinB = (__bf16 *)(w + pl.hinB);
    const int Hs = p.nheads, G = p.ngroups, Bn = (int)p.batch;
    const uint32_t N = (uint32_t)p.N, Lpad = (uint32_t)(p.nch * Q);
    const uint32_t T = (uint32_t)p.T, H = (uint32_t)p.H, W = (uint32_t)p.W;
    const __bf16 *x = (const __bf16 *)a.x, *Bm = (const __bf16 *)a.b, *Cm = (const __bf16 *)a.c;

    if (p.R > 0) {
        bf16_t *rx = (bf16_t *)(w + pl.rx), *rB = (bf16_t *)(w + pl.rB);
        float *rdt = (float *)(w + pl.rdt), *rdtT = (float *)(w + pl.rdtT), *rcsT = (float *)(w + pl.rcsT);
        const uint32_t R = (uint32_t)p.R, Rpad = (uint32_t)(p.nchR * Q);
        const int64_t Cx = (int64_t)Hs * P, Cb = (int64_t)G * S;
        {
            timing::Scope ts_(K_SSD_POOL, st);
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
                ssd::k_pool_f32x4<<<dim3(R, Bn), 256, 0, st>>>(a.dt, rdt, Hs, T, H, W, p.pool_t, p.pool_h, p.pool_w,
                                                              p.order);
            else
                ssd::k_pool<float, float><<<dim3((Hs + 255) / 256, R, Bn), 256, 0, st>>>(
                    a.dt, rdt, Hs, T, H, W, p.pool_t, p.pool_h, p.pool_w, p.order);
        }
        {
            timing::Scope ts_(K_SSD_PREP, st);
            ssd::k_prep_dt<false><<<dim3(p.nchR, (Hs + 63) / 64, Bn), 256, 0, st>>>(rdt, a.a, rdtT, rcsT, Hs, R, Rpad,
                                                                                    Q, 0, 1, 1, R);
        }
        const uint64_t items = (uint64_t)Bn * Hs;
        {
            timing::Scope ts_(K_SSD_STATES, st);
            k_states<S, Q, false><<<grid_of(items), Q * 4, 0, st>>>((const __bf16 *)rx, (const __bf16 *)rB, nullptr, nullptr,
                                                                 rdtT, rcsT,
                                                          a.a, nullptr, nullptr, segF, segB, segA, Hs, G, R, Rpad,
                                                          p.nchR, p.nchR, 1, pl.nseg, pl.nsegT, (uint32_t)items);
        }
    }
    {
        timing::Scope ts_(K_SSD_PREP, st);
        k_perm<<<(N + 255) / 256, 256, 0, st>>>(perm, N, p.order, T, H, W);
    }
    {
        timing::Scope ts_(K_SSD_PREP, st);
        ssd::k_prep_dt<true><<<dim3(p.nch, (Hs + 63) / 64, Bn), 256, 0, st>>>(a.dt, a.a, dtT, csT, Hs, N, Lpad, Q,
                                                                             p.order, T, H, W, perm);
    }
    {
        timing::Scope ts_(K_SSD_CB, st);
        k_cb<S, Q><<<dim3(p.nch, G, Bn), NT, 0, st>>>(Bm, Cm, perm, cb, b16, cfrag, G, N);
    }
    const uint64_t items = (uint64_t)Bn * pl.nseg * Hs;
    {
        timing::Scope ts_(K_SSD_STATES, st);
        k_states<S, Q, true><<<grid_of(items), Q * 4, 0, st>>>(x, Bm, b16, perm, dtT, csT, a.a, hbl, delta, segF, segB, segA, Hs, G,
                                                      N, Lpad, p.nch, pl.segch, pl.nseg, 0, pl.nsegT, (uint32_t)items);
    }
    {
        timing::Scope ts_(K_SSD_SEG_PASS, st);
        k_seg_pass<<<dim3((P * S + 255) / 256, Hs, Bn), 256, 0, st>>>(segF, segB, segA, hinF, hinB, P * S, pl.nseg,
                                                                      pl.nsegT, p.R > 0 ? 1 : 0);
    }
    if (before_out) {
        const hipError_t e = hipStreamWaitEvent(st, before_out, 0);
        if (e != hipSuccess) return e;
    }
    {
        timing::Scope ts_(K_SSD_OUT, st);
        k_out<S, Q><<<grid_of(items), Q * 4, 0, st>>>(x, b16, cfrag, cb, perm, dtT, csT, a.a, a.d, hbl, delta, hinF,
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

hipError_t ssd_fast(const SsdProblem &p, const SsdArgs &a, void *ws, hipStream_t st, hipEvent_t before_out)
{
    if (p.d_state == 128 && p.chunk == 128) return run<128, 128>(p, a, ws, st, before_out);
    if (p.d_state == 64 && p.chunk == 64) return run<64, 64>(p, a, ws, st, before_out);
    if (p.d_state == 128 && p.chunk == 64) return run<128, 64>(p, a, ws, st, before_out);
    return run<64, 128>(p, a, ws, st, before_out);
}

hipError_t ssd_fast_prepare() { return hipSuccess; }

} // namespace mate
