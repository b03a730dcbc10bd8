// Rotary Major Scan reorder: a whole-row gather (canonical -> scan order) or
// scatter (scan order -> canonical) of token rows. Pure HBM streaming: every
// row is read once and written once with the widest aligned vector type.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace mate {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One wave per row, lanes striding over the row's vectors (rows of >= 64 vectors).
template <typename V, bool INV>
__global__ __launch_bounds__(256) void rms_rows_wave(const V *__restrict__ src, V *__restrict__ dst,
                                                     uint32_t N, uint32_t vpr, uint32_t total_rows,
                                                     int order, int flip, uint32_t T, uint32_t H, uint32_t W)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    for (uint32_t r = blockIdx.x * 4u + wave; r < total_rows; r += gridDim.x * 4u) {
        const uint32_t b = r / N, i = r - b * N;
        const uint32_t n = rms_index32(flip ? N - 1u - i : i, order, T, H, W);
        const size_t srow = (size_t)b * N + (INV ? i : n);
        const size_t drow = (size_t)b * N + (INV ? n : i);
        const V *s = src + srow * vpr;
        V *d = dst + drow * vpr;
        uint32_t c = lane;
        for (; c + 448u < vpr; c += 512u) {
            V a[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) a[k] = __builtin_nontemporal_load(s + c + 64u * k);
#pragma unroll
            for (int k = 0; k < 8; ++k) __builtin_nontemporal_store(a[k], d + c + 64u * k);
        }
        for (; c < vpr; c += 64u) __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
    }
}

// Several rows per wave: 2^lg threads per row (rows of < 64 vectors).
template <typename V, bool INV>
__global__ __launch_bounds__(256) void rms_rows_small(const V *__restrict__ src, V *__restrict__ dst,
                                                      uint32_t N, uint32_t vpr, uint32_t total_rows, int lg,
                                                      int order, int flip, uint32_t T, uint32_t H, uint32_t W)
{
    const uint32_t c = threadIdx.x & ((1u << lg) - 1u);
    const uint32_t rows_per_block = 256u >> lg;
    for (uint32_t r = blockIdx.x * rows_per_block + (threadIdx.x >> lg); r < total_rows;
         r += gridDim.x * rows_per_block) {
        if (c >= vpr) continue;
        const uint32_t b = r / N, i = r - b * N;
        const uint32_t n = rms_index32(flip ? N - 1u - i : i, order, T, H, W);
        const size_t srow = (size_t)b * N + (INV ? i : n);
        const size_t drow = (size_t)b * N + (INV ? n : i);
        dst[drow * vpr + c] = src[srow * vpr + c];
    }
}

template <typename V>
hipError_t launch_typed(const void *src, void *dst, uint32_t batch, uint32_t T, uint32_t H, uint32_t W,
                        uint32_t vpr, int order, int flip, int inverse, hipStream_t stream)
{
    const uint32_t N = T * H * W;
    const uint32_t total = batch * N;
    const V *s = (const V *)src;
    V *d = (V *)dst;
    if (vpr >= 64) {
        // The kernel strides over rows, so the grid is capped: a few rounds of resident blocks on
        // every CU, far below the launch limit for any row count the ABI accepts.
        uint32_t blocks = (total + 3u) / 4u;
        if (blocks > 65536u) blocks = 65536u;
        if (inverse)
            rms_rows_wave<V, true><<<blocks, 256, 0, stream>>>(s, d, N, vpr, total, order, flip, T, H, W);
        else
            rms_rows_wave<V, false><<<blocks, 256, 0, stream>>>(s, d, N, vpr, total, order, flip, T, H, W);
    } else {
        int lg = 0;
        while ((1u << lg) < vpr) ++lg;
        const uint32_t rpb = 256u >> lg;
        uint32_t blocks = (total + rpb - 1u) / rpb;
        if (blocks > 8192u) blocks = 8192u;
        if (inverse)
            rms_rows_small<V, true><<<blocks, 256, 0, stream>>>(s, d, N, vpr, total, lg, order, flip, T, H, W);
        else
            rms_rows_small<V, false><<<blocks, 256, 0, stream>>>(s, d, N, vpr, total, lg, order, flip, T, H, W);
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_rms_reorder(const void *src, void *dst, int64_t batch, int64_t T, int64_t H, int64_t W,
                              int64_t row_bytes, int order, int flip, int inverse, hipStream_t stream)
{
    // Widest element that divides the row and both base addresses.
    uintptr_t align = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)row_bytes;
    int64_t e = 16;
    while (e > 1 && (align & (uintptr_t)(e - 1))) e >>= 1;
    const uint32_t vpr = (uint32_t)(row_bytes / e);
    const uint32_t b = (uint32_t)batch, t = (uint32_t)T, h = (uint32_t)H, w = (uint32_t)W;
    timing::Scope ts_(K_RMS_REORDER, stream);
    switch (e) {
    case 16: return launch_typed<u32x4>(src, dst, b, t, h, w, vpr, order, flip, inverse, stream);
    case 8: return launch_typed<u32x2>(src, dst, b, t, h, w, vpr, order, flip, inverse, stream);
    case 4: return launch_typed<uint32_t>(src, dst, b, t, h, w, vpr, order, flip, inverse, stream);
    case 2: return launch_typed<uint16_t>(src, dst, b, t, h, w, vpr, order, flip, inverse, stream);
    default: return launch_typed<uint8_t>(src, dst, b, t, h, w, vpr, order, flip, inverse, stream);
    }
}

} // namespace mate
