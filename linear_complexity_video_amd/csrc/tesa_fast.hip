// TESA on bf16 MFMA (gfx950, v_mfma_f32_32x32x16_bf16), flash-style inside
// each (shifted) 3D window.
//
// Work item = (window, head, block of 256 queries). One persistent workgroup
// of 8 waves per CU runs a sequence of items, each wave 32 queries of the
// current one. The canonical token of every window position is tabulated in
// LDS two items ahead. Keys and values stream through LDS in tiles of 64
// (double buffered, both in their natural row layout; the V^T operand is read
// with the gfx950 LDS transpose read), loaded two tiles ahead through two
// register sets, and the tile stream runs on across items: the next item's
// first tiles load during the current one's last, and its Q rows once the
// last tile's score products are issued (the Q fragments are then free).
// Per tile each wave computes S^T = K Q^T, so that a lane holds one query's
// scores and the softmax needs only one cross-lane exchange; exp'd
// P^T is then directly the B operand of O^T += V^T P^T, and O^T again has one
// query per lane, so the online-softmax rescale is a per-lane multiply. The
// exponent base is the first tile's maximum and is raised (with the rescale)
// only when a later tile's probabilities reach 2^20, so most tiles compute no
// maximum at all. O leaves through a per-wave LDS staging area as whole row
// segments, so moving to the next item needs no barrier. Each XCD owns a
// contiguous range of windows, and the query blocks of one window run side by
// side on adjacent workgroups of that XCD and share its K/V in L2.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "tesa_common.hpp"
#include "timing.hpp"

namespace mate {

namespace {

constexpr int KT = 64;            // keys per LDS tile
constexpr int QW = 32;            // queries per wave
constexpr int NWAVE = 8;          // waves per workgroup
constexpr int QB = QW * NWAVE;    // queries per workgroup
constexpr int KPAD = 8;           // K tile row padding (bf16)
constexpr int VPAD = 32;          // V tile row padding (bf16): spreads transpose reads over the banks

constexpr int MAXW = 4096;        // largest window (tokens) of the MFMA kernel
constexpr int SMALLW = 512;       // windows up to this size take a table ring of this width

template <int DH, int ROWS>
struct __attribute__((aligned(16))) Smem {
    __bf16 k[2][KT][DH + KPAD];
    __bf16 v[2][KT][DH + VPAD];
    __bf16 ostage[8][32 * (DH == 128 ? 64 : 32)];  // per wave: output rows on their way out
    uint32_t row[ROWS];           // canonical token of each window position
};

// One work item: a (batch, head, region, query block) and what the kernel
// derives from it.
struct Item {
    int m;            // tokens in the region
    int q_base;       // first query of the block
    int t0, h0, w0, nt, nh, nw;
    size_t head_off;  // element offset of (batch, head) in q, k, v, o
};

// WHOLE: one window spanning the whole unshifted grid (full attention); a
// window position is then its canonical token, and no table is kept. TW: the
// width of each of the three window tables (the largest window it serves).
//
// Persistent: each workgroup runs a sequence of items. The tiles of
// consecutive items form one stream, so during an item's last key tile the
// next item's first tile and its Q fragments are already loading, and its
// window table is built one item ahead.
template <int DH, bool WHOLE, int TW>
__global__ __launch_bounds__(512) void k_tesa_fast(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                                                   const __bf16 *__restrict__ v, __bf16 *__restrict__ o,
                                                   int nheads, int Tn, int Hn, int Wn, int wt, int wh, int ww,
                                                   int st, int sh, int sw, int nrt, int nrh, int nrw, int nqb,
                                                   uint32_t total, float c_log2)
{
    __shared__ Smem<DH, WHOLE ? 4 : 3 * TW> sm;
    constexpr int DC = DH / 8;  // 16-byte chunks per row

    // Item sequence of this workgroup. Block L runs on XCD L % 8, and XCD x owns a contiguous range of
    // windows (batch, head, region). When the query blocks of a window (nqb of them) divide the XCD's
    // workgroups into groups, each group takes a contiguous run of the range's windows, and its members
    // take one query block of each window, side by side, so that the blocks of a window share its K/V
    // in L2; which member takes which block rotates from window to window, so that windows with fewer
    // blocks (the narrower edge regions of shifted windows) spread their work over the whole group.
    // Otherwise (few windows, many blocks each) the XCD's items (window, query block) are taken in turn.
    const uint32_t wpx = gridDim.x / 8;
    const uint32_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const uint32_t nwin = total / nqb;
    const bool grouped = (uint32_t)nqb <= wpx && wpx % nqb == 0 && nwin >= gridDim.x / nqb;
    const uint32_t G = grouped ? nqb : 1, ng = wpx / G, side = slot % G;
    const uint32_t per_x = grouped ? (nwin + 7) / 8 : (total + 7) / 8;   // windows or items per XCD
    const uint32_t x_hi = min(grouped ? nwin : total, (xcd + 1) * per_x);
    const uint32_t cw = grouped ? (per_x + ng - 1) / ng : 0;            // windows per group
    const uint32_t x_end = grouped ? min(x_hi, xcd * per_x + (slot / G + 1) * cw) : x_hi;
    uint32_t u_next = grouped ? min(x_end, xcd * per_x + (slot / G) * cw) : xcd * per_x + slot;
    const uint32_t u_step = grouped ? 1 : wpx;

    const size_t N = (size_t)Tn * Hn * Wn;
    const size_t rowstride = (size_t)nheads * DH;
    const int nreg = nrt * nrh * nrw;
    // Next item of the sequence with queries in it (false when none is left).
    auto next_item = [&](Item &I) -> bool {
        for (; u_next < x_end; u_next += u_step) {
            const uint32_t win = grouped ? u_next : u_next / nqb;
            const int qb = grouped ? (int)((side + u_next) % G) : (int)(u_next % nqb);
            const int r = win % nreg;
            const int bh = win / nreg;
            const int h = bh % nheads, b = bh / nheads;
            const int rw = r % nrw, rh = (r / nrw) % nrh, rt = r / (nrw * nrh);
            int t0, t1, h0, h1, w0, w1;
            region_extent(rt, Tn, wt, st, t0, t1);
            region_extent(rh, Hn, wh, sh, h0, h1);
            region_extent(rw, Wn, ww, sw, w0, w1);
            I.nt = t1 - t0;
            I.nh = h1 - h0;
            I.nw = w1 - w0;
            I.m = I.nt * I.nh * I.nw;
            I.q_base = qb * QB;
            I.t0 = t0;
            I.h0 = h0;
            I.w0 = w0;
            I.head_off = ((size_t)b * N) * rowstride + (size_t)h * DH;
            if (I.q_base < I.m) {
                u_next += u_step;
                return true;
            }
        }
        return false;
    };

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, col = lane & 31;
    // Canonical token of every window position, in table tb (0 or 1).
    auto build_table = [&](const Item &I, int tb) {
        if (!WHOLE) {
            const int nhw = I.nh * I.nw;
            const float inv_hw = 1.f / (float)nhw, inv_w = 1.f / (float)I.nw;
            for (int l = tid; l < I.m; l += 512) {
                const int lt = div_small(l, nhw, inv_hw);
                const int rem = l - lt * nhw;
                const int lh = div_small(rem, I.nw, inv_w);
                const int lw = rem - lh * I.nw;
                sm.row[tb * TW + l] = (uint32_t)(((I.t0 + lt) * Hn + (I.h0 + lh)) * Wn + (I.w0 + lw));
            }
        }
    };
    auto row_of = [&](int tb, int l) -> size_t { return WHOLE ? (size_t)l : (size_t)sm.row[tb * TW + l]; };

    // Q^T fragments (B operand of S^T = K Q^T) of this lane's query: d = 16 kb + 8 half + 0..7.
    // A query past the window reads the window's first row (finite; its output is never stored),
    // so the loaded values are used as they are and the wait for them falls at their first use.
    auto load_q = [&](const Item &I, int tb, bf16x8 (&qf)[DH / 16]) {
        const int qi = I.q_base + wave * QW + col;
        const __bf16 *qrow = q + I.head_off + row_of(tb, qi < I.m ? qi : 0) * rowstride;
#pragma unroll
        for (int kb = 0; kb < DH / 16; ++kb)
            qf[kb] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qrow + 16 * kb + 8 * half));
    };

    // Items run in sequence; item number s keeps its window table in table s % 3.
    Item I, J, K;
    bool has_j = false, has_k = false;
    int rt = 0;                 // table of the current item
    auto nxt = [](int t) { return t == 2 ? 0 : t + 1; };
    // The next item's Q rows (or the current ones again when none is left: the load is always issued).
    auto load_q_next = [&](bf16x8 (&qf)[DH / 16]) { load_q(has_j ? J : I, has_j ? nxt(rt) : rt, qf); };

    // Tile loader: K and V rows as 16-byte chunks, natural layout.
    constexpr int KCH = KT * DC;                  // chunks per tile
    constexpr int KPER = KCH / 512;               // per thread
    static_assert(KCH % 512 == 0, "tile chunks must split evenly over the workgroup");
    auto fetch = [&](const Item &X, int tb, int kt, u32x4 (&kreg)[KPER], u32x4 (&vreg)[KPER]) {
#pragma unroll
        for (int it = 0; it < KPER; ++it) {
            const int c = tid + 512 * it;
            const int jj = c / DC, dc = c % DC;
            const int kidx = kt * KT + jj;
            // A key past the window reads the window's first key: finite, and its score is masked.
            const size_t off = X.head_off + row_of(tb, kidx < X.m ? kidx : 0) * rowstride + 8 * dc;
            kreg[it] = *(const u32x4 *)(k + off);
            vreg[it] = *(const u32x4 *)(v + off);
        }
    };
    auto stash = [&](int b, const u32x4 (&kreg)[KPER], const u32x4 (&vreg)[KPER]) {
#pragma unroll
        for (int it = 0; it < KPER; ++it) {
            const int c = tid + 512 * it;
            *(u32x4 *)&sm.k[b][c / DC][8 * (c % DC)] = kreg[it];
            *(u32x4 *)&sm.v[b][c / DC][8 * (c % DC)] = vreg[it];
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

    // One key tile of the current item from LDS buffer b: S^T, softmax, O^T.
    auto compute = [&](const Item &X, int kt, int b, bf16x8 (&qf)[DH / 16], f32x16 (&acc)[DH / 32],
                       float &mrun, float &lrun, bool last) {
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int kb = 0; kb < DH / 16; ++kb) {
                const bf16x8 a = *(const bf16x8 *)&sm.k[b][32 * sub + col][16 * kb + 8 * half];
                s[sub] = mfma(a, qf[kb], s[sub]);
            }
        // After the item's last score products, the next item's Q rows load into the fragments
        // while this tile's softmax and P V run.
        if (last) load_q_next(qf);
        // Keys past the window (only in the last, ragged tile) get -inf.
        if (kt * KT + KT > X.m) {
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int j = kt * KT + 32 * sub + 8 * (rr >> 2) + 4 * half + (rr & 3);
                    s[sub][rr] = j < X.m ? s[sub][rr] : -INFINITY;
                }
        }
        // Probabilities against the base mrun (log2 units): the exact maximum of the
        // first tile, raised later only when a tile's probabilities reach 2^20 (or
        // overflow): then O and l are rescaled and the tile's probabilities recomputed.
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
                acc[dt] = mfma(v_frag<DH + VPAD>(&sm.v[b][0][0], 16 * kb2, 32 * dt), pf[kb2], acc[dt]);
    };

    // Tiles of an item, rounded up to even: a tile's LDS buffer and register set
    // follow its parity. A padded tile holds no key and skips the arithmetic.
    auto tiles_of = [](const Item &X) {
        const int n = (X.m + KT - 1) / KT;
        return n + (n & 1);
    };

    // The table (and the decode) of the item after the next one is made during
    // the current item's first tile pair, after that pair's first barrier: by
    // then every wave has finished the item that used the same table.
    if (!next_item(I)) return;  // uniform over the workgroup
    has_j = next_item(J);
    build_table(I, rt);
    if (has_j) build_table(J, nxt(rt));
    __syncthreads();
    bf16x8 qf[DH / 16];
    load_q(I, rt, qf);
    // Two tiles in flight: set 0 carries even tiles, set 1 odd ones.
    u32x4 k0[KPER], v0[KPER], k1[KPER], v1[KPER];
    fetch(I, rt, 0, k0, v0);
    fetch(I, rt, 1, k1, v1);
    stash(0, k0, v0);
    __syncthreads();

    // Stream position kt of the current item (n tiles); past its end the next
    // item's tile kt - n; with nothing left the current item's tile 0 again.
    // Every fetch is issued, so the compiler's memory waits stay exact.
    auto fetch_pos = [&](int kt, int n, u32x4 (&kreg)[KPER], u32x4 (&vreg)[KPER]) {
        const bool in_i = kt < n, use_j = !in_i && has_j;
        fetch(use_j ? J : I, use_j ? nxt(rt) : rt, in_i ? kt : (use_j ? kt - n : 0), kreg, vreg);
    };

    for (;;) {
        const bool wave_active = I.q_base + wave * QW < I.m;
        const int n = tiles_of(I);
        f32x16 acc[DH / 32];
#pragma unroll
        for (int i = 0; i < DH / 32; ++i) acc[i] = f32x16{};
        float mrun = 0.f, lrun = 0.f;
        const int last_kt = (I.m + KT - 1) / KT - 1;  // the item's last tile with keys
        for (int kt = 0; kt < n; kt += 2) {
            // even tile kt (buffer 0); tile kt + 1 waits in set 1, tile kt + 2 goes to set 0
            fetch_pos(kt + 2, n, k0, v0);
            if (wave_active && kt * KT < I.m) compute(I, kt, 0, qf, acc, mrun, lrun, kt == last_kt);
            stash(1, k1, v1);
            __syncthreads();
            // odd tile kt + 1 (buffer 1); tile kt + 2 waits in set 0, tile kt + 3 goes to set 1
            fetch_pos(kt + 3, n, k1, v1);
            if (kt == 0 && has_j) {
                has_k = next_item(K);
                if (has_k) build_table(K, nxt(nxt(rt)));
            }
            if (wave_active && (kt + 1) * KT < I.m) compute(I, kt + 1, 1, qf, acc, mrun, lrun, kt + 1 == last_kt);
            stash(0, k0, v0);
            __syncthreads();
        }
        // A wave with no queries in this item loads the next item's Q rows here.
        if (!wave_active) load_q_next(qf);

        // O leaves through this wave's staging area, in rounds of RD value dims
        // (16-byte chunks XOR-swizzled by row against bank conflicts): all rows are
        // read back first, then stored as whole row segments by consecutive lanes.
        {
            constexpr int RD = DH == 128 ? 64 : 32;  // value dims per round
            constexpr int CPR = RD / 8;              // 16-byte chunks per row segment
            constexpr int PER = 32 * CPR / 64;       // chunks per lane and round
            __bf16 *stage = sm.ostage[wave];
            const float inv = 1.f / (lrun + __shfl_xor(lrun, 32));
            size_t dst[PER];
            bool ok[PER];
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int rq = (lane + 64 * j) / CPR, qq = I.q_base + wave * QW + rq;
                ok[j] = qq < I.m;
                dst[j] = I.head_off + row_of(rt, ok[j] ? qq : 0) * rowstride + 8 * ((lane + 64 * j) % CPR);
            }
            u32x4 val[DH / RD][PER];
#pragma unroll
            for (int r = 0; r < DH / RD; ++r) {
#pragma unroll
                for (int d2 = 0; d2 < RD / 32; ++d2)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        bf16x4 out;
#pragma unroll
                        for (int i = 0; i < 4; ++i) out[i] = (__bf16)(acc[r * (RD / 32) + d2][4 * g + i] * inv);
                        const int ch = (4 * d2 + g) ^ (col & (CPR - 1));
                        *(bf16x4 *)(stage + col * RD + 8 * ch + 4 * half) = out;
                    }
#pragma unroll
                for (int j = 0; j < PER; ++j) {
                    const int idx = lane + 64 * j, rq = idx / CPR, ch = idx % CPR;
                    val[r][j] = *(const u32x4 *)(stage + rq * RD + 8 * (ch ^ (rq & (CPR - 1))));
                }
            }
#pragma unroll
            for (int r = 0; r < DH / RD; ++r)
#pragma unroll
                for (int j = 0; j < PER; ++j)
                    if (ok[j]) *(u32x4 *)(o + dst[j] + RD * r) = val[r][j];
        }
        if (!has_j) break;
        I = J;
        J = K;
        has_j = has_k;
        has_k = false;
        rt = nxt(rt);
    }
}

int cu_count()
{
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int DH, bool WHOLE, int TW>
hipError_t launch(const TesaProblem &p, const TesaArgs &a, hipStream_t stream)
{
    const int maxw = p.wt * p.wh * p.ww;
    const int nqb = (maxw + QB - 1) / QB;
    const uint64_t total = (uint64_t)p.batch * p.nheads * p.nrt * p.nrh * p.nrw * nqb;
    // One workgroup per CU (its LDS or its registers leave no room for a second), a multiple of 8 (one set
    // per XCD).
    const uint64_t want = ((uint64_t)cu_count() + 7) / 8 * 8;
    const uint64_t blocks = std::min<uint64_t>(want, (total + 7) / 8 * 8);
    const float scale = p.scale > 0.f ? p.scale : 1.f / sqrtf((float)DH);
    timing::Scope ts_(K_TESA, stream);
    k_tesa_fast<DH, WHOLE, TW><<<dim3((unsigned)blocks), dim3(512), 0, stream>>>(
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
    const bool small = (int64_t)p.wt * p.wh * p.ww <= SMALLW;
    if (p.headdim == 64) {
        if (whole) return launch<64, true, 1>(p, a, stream);
        return small ? launch<64, false, SMALLW>(p, a, stream) : launch<64, false, MAXW>(p, a, stream);
    }
    if (whole) return launch<128, true, 1>(p, a, stream);
    return small ? launch<128, false, SMALLW>(p, a, stream) : launch<128, false, MAXW>(p, a, stream);
}

} // namespace mate
