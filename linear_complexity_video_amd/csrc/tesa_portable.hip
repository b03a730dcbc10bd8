// Portable TESA kernel (fp32 FMA): one workgroup per (window, head, batch),
// one thread per query, keys streamed through LDS in tiles of 32 with an
// online softmax. Used for fp32 tensors and head sizes without MFMA kernels.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace mate {

namespace {

// Extent of region r along an axis of length D with window w and shift s:
// region ids follow (c + w - s) div w, so with s > 0 the first region is
// [0, s) and the following ones start at s, s + w, ...
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

template <typename T, int DH>
__global__ __launch_bounds__(256) void k_tesa_portable(const T *__restrict__ q, const T *__restrict__ k,
                                                       const T *__restrict__ v, T *__restrict__ o, int nheads,
                                                       int Tn, int Hn, int Wn, int wt, int wh, int ww, int st,
                                                       int sh, int sw, int nrh, int nrw, float scale)
{
    constexpr int KT = 32;
    __shared__ float Ks[KT][DH + 1];
    __shared__ float Vs[KT][DH + 1];
    const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int rw = r % nrw, rh = (r / nrw) % nrh, rt = r / (nrw * nrh);
    int t0, t1, h0, h1, w0, w1;
    region_extent(rt, Tn, wt, st, t0, t1);
    region_extent(rh, Hn, wh, sh, h0, h1);
    region_extent(rw, Wn, ww, sw, w0, w1);
    const int nt = t1 - t0, nh = h1 - h0, nw = w1 - w0, m = nt * nh * nw;
    const size_t N = (size_t)Tn * Hn * Wn;
    auto token = [&](int l) -> size_t {
        const int lw = l % nw, lh = (l / nw) % nh, lt = l / (nw * nh);
        return ((size_t)(t0 + lt) * Hn + (h0 + lh)) * Wn + (w0 + lw);
    };
    for (int q0 = 0; q0 < m; q0 += 256) {
        const int qi = q0 + threadIdx.x;
        const bool active = qi < m;
        float qv[DH], acc[DH];
        size_t qrow = 0;
        if (active) {
            qrow = (((size_t)b * N + token(qi)) * nheads + h) * DH;
#pragma unroll
            for (int e = 0; e < DH; ++e) qv[e] = elem<T>::load(q + qrow + e) * scale;
        }
#pragma unroll
        for (int e = 0; e < DH; ++e) acc[e] = 0.f;
        float mx = -INFINITY, l = 0.f;
        for (int k0 = 0; k0 < m; k0 += KT) {
            __syncthreads();
            for (int idx = threadIdx.x; idx < KT * DH; idx += 256) {
                const int j = idx / DH, e = idx - j * DH;
                float kv = 0.f, vv = 0.f;
                if (k0 + j < m) {
                    const size_t off = (((size_t)b * N + token(k0 + j)) * nheads + h) * DH + e;
                    kv = elem<T>::load(k + off);
                    vv = elem<T>::load(v + off);
                }
                Ks[j][e] = kv;
                Vs[j][e] = vv;
            }
            __syncthreads();
            if (!active) continue;
            const int nk = min(KT, m - k0);
            float s[KT];
            float bm = -INFINITY;
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                float a = 0.f;
#pragma unroll
                for (int e = 0; e < DH; ++e) a += qv[e] * Ks[j][e];
                s[j] = j < nk ? a : -INFINITY;
                bm = fmaxf(bm, s[j]);
            }
            const float nm = fmaxf(mx, bm);
            const float corr = __expf(mx - nm);
            l *= corr;
#pragma unroll
            for (int e = 0; e < DH; ++e) acc[e] *= corr;
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                const float pj = j < nk ? __expf(s[j] - nm) : 0.f;
                l += pj;
#pragma unroll
                for (int e = 0; e < DH; ++e) acc[e] += pj * Vs[j][e];
            }
            mx = nm;
        }
        if (active) {
            const float inv = 1.f / l;
#pragma unroll
            for (int e = 0; e < DH; ++e) elem<T>::store(o + qrow + e, acc[e] * inv);
        }
    }
}

template <typename T, int DH>
hipError_t launch_dh(const TesaProblem &p, const TesaArgs &a, hipStream_t st)
{
    const float scale = p.scale > 0.f ? p.scale : 1.f / sqrtf((float)DH);
    dim3 grid((unsigned)(p.nrt * p.nrh * p.nrw), (unsigned)p.nheads, (unsigned)p.batch);
    timing::Scope ts_(K_TESA, st);
    k_tesa_portable<T, DH><<<grid, 256, 0, st>>>((const T *)a.q, (const T *)a.k, (const T *)a.v, (T *)a.o,
                                                  p.nheads, (int)p.T, (int)p.H, (int)p.W, p.wt, p.wh, p.ww, p.st,
                                                  p.sh, p.sw, p.nrh, p.nrw, scale);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const TesaProblem &p, const TesaArgs &a, hipStream_t st)
{
    switch (p.headdim) {
    case 8: return launch_dh<T, 8>(p, a, st);
    case 16: return launch_dh<T, 16>(p, a, st);
    case 32: return launch_dh<T, 32>(p, a, st);
    case 64: return launch_dh<T, 64>(p, a, st);
    case 128: return launch_dh<T, 128>(p, a, st);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

bool tesa_portable_supports(const TesaProblem &p)
{
    const int dh = p.headdim;
    return (dh == 8 || dh == 16 || dh == 32 || dh == 64 || dh == 128) && p.wt * p.wh * p.ww <= 1024;
}

hipError_t tesa_portable(const TesaProblem &p, const TesaArgs &a, hipStream_t st)
{
    if (p.dtype == 0) return launch_t<float>(p, a, st);
    return launch_t<bf16_t>(p, a, st);
}

} // namespace mate
