// Device-side helpers shared by the MATE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mate {

// bfloat16 is carried as its 16-bit pattern; arithmetic is always fp32.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

template <typename T> struct elem;
template <> struct elem<float> {
    __device__ __forceinline__ static float load(const float *p) { return *p; }
    __device__ __forceinline__ static void store(float *p, float v) { *p = v; }
};
template <> struct elem<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t *p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void store(bf16_t *p, float v) { *p = f32_to_bf16(v); }
};

// Rotary Major Scan: canonical token index of scan position i (0 <= i < T*H*W)
// for unroll order `order`, loops written outermost first:
//   0: t,h,w   1: t,w,h   2: h,w,t   3: w,h,t
// Order 4 is the zigzag (snake) path that RMS replaces (QbitAI article, section
// "方法"; xllm-io review, Table 2): frame t runs its rows forward on even t and
// backward on odd t, and row k of the path (k = t*H + position in the frame)
// runs along w forward on even k and backward on odd k, so consecutive tokens
// are grid neighbours.
__device__ __forceinline__ int64_t rms_index(int64_t i, int order, int64_t T, int64_t H, int64_t W)
{
    int64_t t, h, w;
    switch (order) {
    case 0:
        return i;
    case 1: {
        t = i / (W * H);
        int64_t r = i - t * (W * H);
        w = r / H;
        h = r - w * H;
        break;
    }
    case 2: {
        h = i / (W * T);
        int64_t r = i - h * (W * T);
        w = r / T;
        t = r - w * T;
        break;
    }
    case 3: {
        w = i / (H * T);
        int64_t r = i - w * (H * T);
        h = r / T;
        t = r - h * T;
        break;
    }
    default: {
        const int64_t k = i / W;  // row of the path
        const int64_t c = i - k * W;
        t = k / H;
        const int64_t r = k - t * H;
        h = (t & 1) ? H - 1 - r : r;
        w = (k & 1) ? W - 1 - c : c;
        break;
    }
    }
    return (t * H + h) * W + w;
}

// 32-bit variant for grids with fewer than 2^31 tokens (every launch checks).
__device__ __forceinline__ uint32_t rms_index32(uint32_t i, int order, uint32_t T, uint32_t H, uint32_t W)
{
    uint32_t t, h, w;
    switch (order) {
    case 0:
        return i;
    case 1: {
        t = i / (W * H);
        uint32_t r = i - t * (W * H);
        w = r / H;
        h = r - w * H;
        break;
    }
    case 2: {
        h = i / (W * T);
        uint32_t r = i - h * (W * T);
        w = r / T;
        t = r - w * T;
        break;
    }
    case 3: {
        w = i / (H * T);
        uint32_t r = i - w * (H * T);
        h = r / T;
        t = r - h * T;
        break;
    }
    default: {
        const uint32_t k = i / W;  // row of the path
        const uint32_t c = i - k * W;
        t = k / H;
        const uint32_t r = k - t * H;
        h = (t & 1u) ? H - 1u - r : r;
        w = (k & 1u) ? W - 1u - c : c;
        break;
    }
    }
    return (t * H + h) * W + w;
}

} // namespace mate
