// TESA on bf16 MFMA (gfx950, v_mfma_f32_32x32x16_bf16), flash-style inside
// each (shifted) 3D window.
//
// Work item = (window, head, block of 256 queries); a workgroup of 8 waves
// owns one item, each wave 32 queries. The canonical token of every window
// position is tabulated in LDS once per item. Keys and values stream through LDS in
// tiles of 64 (double buffered, both in their natural row layout; the V^T
// operand is read with the gfx950 LDS transpose read). Per tile each wave
// computes S^T = K Q^T, so that a lane holds one query's scores and the
// softmax needs only one cross-lane exchange; exp'd P^T is then directly the
// B operand of O^T += V^T P^T, and O^T again has one query per lane, so the
// online-softmax rescale is a per-lane multiply. The exponent base is the
// first tile's maximum and is raised (with the rescale) only when a later
// tile's probabilities reach 2^20, so most tiles compute no maximum at all. Consecutive block ids are
// spread over the 8 XCDs; they are remapped so that the query blocks of one
// window land on the same XCD and share its K/V in L2.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace mate {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int KT = 64;            // keys per LDS tile
constexpr int QW = 32;            // queries per wave
constexpr int NWAVE = 8;          // waves per workgroup
constexpr int QB = QW * NWAVE;    // queries per workgroup
constexpr int KPAD = 8;           // K tile row padding (bf16)
constexpr int VPAD = 32;          // V tile row padding (bf16): spreads transpose reads over the banks

__device__ __forceinline__ void region_extent(int r, int D, int w, int s, int &lo, int &hi)
{
    if (s == 0) {
        lo = r * w;
        hi = lo + w;
    } else if (r == 0) {
        lo = 0;
        hi = s;
    } else {
        lo = s + (r - 1) * w;
        hi = lo + w;
    }
    if (hi > D) hi = D;
}

constexpr int MAXW = 4096;        // largest window (tokens) of the MFMA kernel

template <int DH, int ROWS>
struct __attribute__((aligned(16))) Smem {
    __bf16 k[2][KT][DH + KPAD];
    __bf16 v[2][KT][DH + VPAD];
    uint32_t row[ROWS];           // canonical token of each window position
};

// A operand of O^T += V^T P^T from the row-major V tile: lane l gets column
// (value dim) n_base + l % 32 at keys k_base + 4 (l / 32) + {0..3} and
// k_base + 8 + 4 (l / 32) + {0..3}, the key order of the P^T fragment.
template <int LD>
__device__ __forceinline__ bf16x8 v_frag(const __bf16 *tile, int k_base, int n_base)
{
    const int l = threadIdx.x & 63, g = l >> 4, s = l & 15;
    const __bf16 *p = tile + (k_base + 4 * (g >> 1) + (s >> 2)) * LD + n_base + 16 * (g & 1) + 4 * (s & 3);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 8 * LD));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// WHOLE: one window spanning the whole unshifted grid (full attention); a
// window position is then its canonical token, and no table is kept.
template <int DH, bool WHOLE>
__global__ __launch_bounds__(512) void k_tesa_fast(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                                                   const __bf16 *__restrict__ v, __bf16 *__restrict__ o,
                                                   int nheads, int Tn, int Hn, int Wn, int wt, int wh, int ww,
                                                   int st, int sh, int sw, int nrt, int nrh, int nrw, int nqb,
                                                   uint32_t total, float c_log2)
{
    __shared__ Smem<DH, WHOLE ? 4 : MAXW> sm;
    constexpr int DC = DH / 8;  // 16-byte chunks per row

    // XCD-aware item index: block L runs on XCD L % 8; items w, w+1, ... of one
    // XCD are consecutive query blocks / windows.
    const uint32_t per_xcd = gridDim.x / 8;
    const uint32_t item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= total) return;
    const int qb = item % nqb;
    const uint32_t rest = item / nqb;
    const int nreg = nrt * nrh * nrw;
    const int r = rest % nreg;
    const int bh = rest / nreg;
    const int h = bh % nheads, b = bh / nheads;
    const int rw = r % nrw, rh = (r / nrw) % nrh, rt = r / (nrw * nrh);
    int t0, t1, h0, h1, w0, w1;
    region_extent(rt, Tn, wt, st, t0, t1);
    region_extent(rh, Hn, wh, sh, h0, h1);
    region_extent(rw, Wn, ww, sw, w0, w1);
    const int nt = t1 - t0, nh_ = h1 - h0, nw_ = w1 - w0, m = nt * nh_ * nw_;
    const int q_base = qb * QB;
    if (q_base >= m) return;  // uniform over the workgroup

    const size_t N = (size_t)Tn * Hn * Wn;
    const size_t rowstride = (size_t)nheads * DH;
    const size_t head_off = ((size_t)b * N) * rowstride + (size_t)h * DH;
    auto token = [&](int l) -> size_t {
        const int lw = l % nw_, lh = (l / nw_) % nh_, lt = l / (nw_ * nh_);
        return ((size_t)(t0 + lt) * Hn + (h0 + lh)) * Wn + (w0 + lw);
    };

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // Canonical token of every window position, computed once (the tile loader only looks it up).
    if (!WHOLE) {
        for (int l = tid; l < m; l += 512) sm.row[l] = (uint32_t)token(l);
        __syncthreads();
    }
    auto row_of = [&](int l) -> size_t { return WHOLE ? (size_t)l : (size_t)sm.row[l]; };
    const int half = lane >> 5, col = lane & 31;
    const int qi = q_base + wave * QW + col;
    const bool qvalid = qi < m;
    const bool wave_active = q_base + wave * QW < m;

    // Q^T fragments (B operand of S^T = K Q^T): query col, d = 16 kb + 8 half + 0..7.
    bf16x8 qf[DH / 16];
    {
        const __bf16 *qrow = q + head_off + row_of(qvalid ? qi : 0) * rowstride;
#pragma unroll
        for (int kb = 0; kb < DH / 16; ++kb) {
            u32x4 raw = qvalid ? *(const u32x4 *)(qrow + 16 * kb + 8 * half) : u32x4{0, 0, 0, 0};
            qf[kb] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    f32x16 acc[DH / 32];
#pragma unroll
    for (int i = 0; i < DH / 32; ++i) acc[i] = f32x16{};
    float mrun = 0.f, lrun = 0.f;
    const int ntiles = (m + KT - 1) / KT;

    // Tile loader: K and V rows as 16-byte chunks, natural layout.
    constexpr int KCH = KT * DC;                  // chunks per tile
    constexpr int KPER = KCH / 512;               // per thread
    static_assert(KCH % 512 == 0, "tile chunks must split evenly over the workgroup");
    u32x4 kreg[KPER], vreg[KPER];
    auto fetch = [&](int kt) {
#pragma unroll
        for (int it = 0; it < KPER; ++it) {
            const int c = tid + 512 * it;
            const int jj = c / DC, dc = c % DC;
            const int kidx = kt * KT + jj;
            // A key past the window reads the window's first key: finite, and its score is masked.
            const size_t off = head_off + row_of(kidx < m ? kidx : 0) * rowstride + 8 * dc;
            kreg[it] = *(const u32x4 *)(k + off);
            vreg[it] = *(const u32x4 *)(v + off);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int it = 0; it < KPER; ++it) {
            const int c = tid + 512 * it;
            *(u32x4 *)&sm.k[buf][c / DC][8 * (c % DC)] = kreg[it];
            *(u32x4 *)&sm.v[buf][c / DC][8 * (c % DC)] = vreg[it];
        }
    };

    // Maximum score of one tile for this lane's query, in log2 units.
    auto tile_max = [&](const f32x16 (&s)[2]) -> float {
        float mloc = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) mloc = fmaxf(mloc, s[sub][rr]);
        return fmaxf(mloc, __shfl_xor(mloc, 32)) * c_log2;
    };
    // P^T fragments of one tile against base m, and this lane's sum of them
    // (of the bf16-rounded values that enter P V).
    auto probs = [&](const f32x16 (&s)[2], float m, bf16x8 (&pf)[4]) -> float {
        float lsum = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2) {
                    bf16x2 p2;
                    p2[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][8 * hb + jj], c_log2, -m));
                    p2[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][8 * hb + jj + 1], c_log2, -m));
                    pf[2 * sub + hb][jj] = p2[0];
                    pf[2 * sub + hb][jj + 1] = p2[1];
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(p2, bf16x2{(__bf16)1.f, (__bf16)1.f}, lsum, false);
                }
        return lsum;
    };

    fetch(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < ntiles) fetch(kt + 1);
        if (wave_active) {
            f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int kb = 0; kb < DH / 16; ++kb) {
                    const bf16x8 a = *(const bf16x8 *)&sm.k[cur][32 * sub + col][16 * kb + 8 * half];
                    s[sub] = mfma(a, qf[kb], s[sub]);
                }
            // Keys past the window (only in the last, ragged tile) get -inf.
            if (kt * KT + KT > m) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        const int j = kt * KT + 32 * sub + 8 * (rr >> 2) + 4 * half + (rr & 3);
                        s[sub][rr] = j < m ? s[sub][rr] : -INFINITY;
                    }
            }
            // Probabilities against the base mrun (log2 units): the exact maximum
            // of the first tile, raised later only when a tile's probabilities
            // reach 2^20 (or overflow): then O and l are rescaled and the tile's
            // probabilities recomputed.
            if (kt == 0) mrun = tile_max(s);
            bf16x8 pf[4];
            float lsum = probs(s, mrun, pf);
            if (__any(!(lsum < 0x1p20f))) {
                const float mnew = fmaxf(mrun, tile_max(s));
                const float corr = __builtin_amdgcn_exp2f(mrun - mnew);
                lrun *= corr;
#pragma unroll
                for (int i = 0; i < DH / 32; ++i) acc[i] *= corr;
                mrun = mnew;
                lsum = probs(s, mrun, pf);
            }
            lrun += lsum;
#pragma unroll
            for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2)
                    acc[dt] = mfma(v_frag<DH + VPAD>(&sm.v[cur][0][0], 16 * kb2, 32 * dt), pf[kb2], acc[dt]);
        }
        if (kt + 1 < ntiles) stash(cur ^ 1);
        __syncthreads();
    }

    const float lt = lrun + __shfl_xor(lrun, 32);
    if (qvalid) {
        const float inv = 1.f / lt;
        __bf16 *orow = o + head_off + row_of(qi) * rowstride;
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 out;
#pragma unroll
                for (int i = 0; i < 4; ++i) out[i] = (__bf16)(acc[dt][4 * g + i] * inv);
                *(bf16x4 *)(orow + 32 * dt + 8 * g + 4 * half) = out;
            }
    }
}

template <int DH, bool WHOLE>
hipError_t launch(const TesaProblem &p, const TesaArgs &a, hipStream_t stream)
{
    const int maxw = p.wt * p.wh * p.ww;
    const int nqb = (maxw + QB - 1) / QB;
    const uint64_t total = (uint64_t)p.batch * p.nheads * p.nrt * p.nrh * p.nrw * nqb;
    const uint64_t blocks = (total + 7) / 8 * 8;
    const float scale = p.scale > 0.f ? p.scale : 1.f / sqrtf((float)DH);
    timing::Scope ts_(K_TESA, stream);
    k_tesa_fast<DH, WHOLE><<<dim3((unsigned)blocks), dim3(512), 0, stream>>>(
        (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v, (__bf16 *)a.o, p.nheads, (int)p.T,
        (int)p.H, (int)p.W, p.wt, p.wh, p.ww, p.st, p.sh, p.sw, p.nrt, p.nrh, p.nrw, nqb, (uint32_t)total,
        scale * 1.4426950408889634f);
    return hipGetLastError();
}

} // namespace

bool tesa_fast_supports(const TesaProblem &p)
{
    const int64_t wsize = (int64_t)p.wt * p.wh * p.ww;
    const bool whole = p.nrt == 1 && p.nrh == 1 && p.nrw == 1;
    const int64_t items = p.batch * p.nheads * (int64_t)p.nrt * p.nrh * p.nrw * ((wsize + QB - 1) / QB);
    return p.dtype == 1 && (p.headdim == 64 || p.headdim == 128) && (whole || wsize <= MAXW) &&
           items < ((int64_t)1 << 30);
}

hipError_t tesa_fast(const TesaProblem &p, const TesaArgs &a, hipStream_t stream)
{
    const bool whole = p.nrt == 1 && p.nrh == 1 && p.nrw == 1;
    if (p.headdim == 64) return whole ? launch<64, true>(p, a, stream) : launch<64, false>(p, a, stream);
    return whole ? launch<128, true>(p, a, stream) : launch<128, false>(p, a, stream);
}

} // namespace mate
