// Internal launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mate {

// Validated bidirectional-SSD problem (derived sizes filled in by the ABI layer).
struct SsdProblem {
    int64_t batch, T, H, W, N;
    int nheads, headdim, d_state, ngroups, chunk, order;
    int pool_t, pool_h, pool_w;
    int64_t R;      // review tokens (0 = none)
    int nch, nchR;  // chunks of the main / review sequence
    int dtype;      // 0 fp32, 1 bf16
};

struct SsdArgs {
    const void *x, *b, *c;
    const float *dt, *a, *d;
    void *y;
};

// Inputs and gradients of the scan's backward (dt, a, d, ddt, da, dd fp32; the rest in the scan's dtype).
struct SsdGradArgs {
    const void *x, *b, *c;
    const float *dt, *a, *d;
    const void *dy;
    void *dx, *db, *dc;
    float *ddt, *da, *dd;
};

struct TesaProblem {
    int64_t batch, T, H, W;
    int nheads, headdim;
    int wt, wh, ww, st, sh, sw;
    int nrt, nrh, nrw;  // regions along each axis
    float scale;
    int dtype;
};

struct TesaArgs {
    const void *q, *k, *v;
    void *o;
};

struct TesaGradArgs {
    const void *q, *k, *v, *dout;
    void *dq, *dk, *dv;
};

// Validated bidirectional Mamba (selective scan) problem.
struct MambaProblem {
    int64_t batch, T, H, W;
    int channels, d_state, order;
    int pool_t, pool_h, pool_w;
    int64_t R;  // review tokens (0 = none)
    int dtype;  // 0 fp32, 1 bf16
};

struct MambaArgs {
    const void *x, *b, *c;
    const float *dt, *a, *d;
    void *y;
};

size_t mamba_workspace(const MambaProblem &p);
hipError_t mamba_scan(const MambaProblem &p, const MambaArgs &a, void *ws, hipStream_t st);

// Device address of the library-held scratch array (MATE_STATIC_SCRATCH_BYTES) on the current
// device, looked up once per device.
hipError_t static_scratch(void **out);

hipError_t launch_rms_reorder(const void *src, void *dst, int64_t batch, int64_t T, int64_t H, int64_t W,
                              int64_t row_bytes, int order, int flip, int inverse, hipStream_t stream);

size_t ssd_portable_workspace(const SsdProblem &p);
hipError_t ssd_portable(const SsdProblem &p, const SsdArgs &a, void *ws, hipStream_t st);
hipError_t ssd_portable_prepare();

bool ssd_fast_supports(const SsdProblem &p);
size_t ssd_fast_workspace(const SsdProblem &p);
hipError_t ssd_fast(const SsdProblem &p, const SsdArgs &a, void *ws, hipStream_t st);
hipError_t ssd_fast_prepare();

bool ssd_backward_supports(const SsdProblem &p);
size_t ssd_backward_workspace(const SsdProblem &p);
hipError_t ssd_backward(const SsdProblem &p, const SsdGradArgs &a, void *ws, hipStream_t st);
hipError_t ssd_backward_prepare();

bool tesa_portable_supports(const TesaProblem &p);
hipError_t tesa_portable(const TesaProblem &p, const TesaArgs &a, hipStream_t st);

bool tesa_fast_supports(const TesaProblem &p);
hipError_t tesa_fast(const TesaProblem &p, const TesaArgs &a, hipStream_t st);

bool tesa_backward_supports(const TesaProblem &p);
size_t tesa_backward_workspace(const TesaProblem &p);
hipError_t tesa_backward(const TesaProblem &p, const TesaGradArgs &a, void *ws, hipStream_t st);

} // namespace mate
