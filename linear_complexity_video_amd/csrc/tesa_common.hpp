// Helpers shared by the TESA forward and backward MFMA kernels (gfx950).
#pragma once

#include "common.hpp"

namespace mate {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Extent [lo, hi) of region r along an axis of extent D, window w and shift s:
// the first region holds s positions when s > 0, the interior ones w.
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

// A operand read transposed from a row-major tile (rows: tokens, columns: head
// dims) with the gfx950 LDS transpose read: lane l gets column n_base + l % 32 at
// rows k_base + 4 (l / 32) + {0..3} and k_base + 8 + 4 (l / 32) + {0..3}, the
// token order in which an accumulator's 16 rows become a B fragment (V^T in the
// forward's O^T += V^T P^T; K^T, Q^T and dO^T in the backward).
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

// a / d for 0 <= a, d < 2^22 from a float reciprocal of d: the estimate is
// within one of the quotient, and one correction step makes it exact.
__device__ __forceinline__ int div_small(int a, int d, float inv_d)
{
    int qt = (int)((float)a * inv_d);
    const int r = a - qt * d;
    qt += (r >= d) - (r < 0);
    return qt;
}

} // namespace
} // namespace mate
