// MFMA operand fragments from LDS tiles (gfx950, wave64), shared by the scan's
// kernels. For v_mfma_f32_32x32x16_bf16 (and the fp16 form), lane l supplies
// A[m = l % 32][k = 8 (l / 32) + 0..7] and B[k = 8 (l / 32) + 0..7][n = l % 32];
// the 16 accumulators of lane l hold C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
// Tiles are bf16, row-major with a row stride `ld` (in elements) that keeps
// every row 16-byte aligned.
#pragma once

#include "common.hpp"

namespace mate {
namespace frag {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Fragment from a row-major [k][n] tile: lane l gets column n_base + l % 32 at
// rows k_base + 8 (l / 32) + 0..7 (two gfx950 LDS transpose reads). This is the
// B operand of a [k][n] tile, or the A operand of a tile stored as [k][m].
__device__ __forceinline__ bf16x8 frag_tr(const __bf16 *tile, int ld, int k_base, int n_base)
{
    const int l = threadIdx.x & 63, g = l >> 4, s = l & 15;
    const __bf16 *p = tile + (k_base + 8 * (g >> 1) + (s >> 2)) * ld + n_base + 16 * (g & 1) + 4 * (s & 3);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * ld));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Fragment from a row-major [m][k] tile: lane l gets row m_base + l % 32 at
// columns k_base + 8 (l / 32) + 0..7 (one 16-byte read). This is the A operand of
// an [m][k] tile, or the B operand of a tile stored as [n][k].
__device__ __forceinline__ bf16x8 frag_rm(const __bf16 *tile, int ld, int m_base, int k_base)
{
    const int l = threadIdx.x & 63;
    return *(const bf16x8 *)(tile + (m_base + (l & 31)) * ld + k_base + 8 * (l >> 5));
}

// Row of accumulator i of lane l inside its 32 x 32 tile (the column is l % 32).
__device__ __forceinline__ int acc_row(int i, int l) { return 8 * (i >> 2) + 4 * (l >> 5) + (i & 3); }

} // namespace frag
} // namespace mate
