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

// One MATE layer around the core (layer.cpp, layer_ops.hip).
struct LayerDims {
    int64_t tokens;  // batch * T * H * W
    int d_model;
    int inner;       // nheads * headdim (x, z, y)
    int bc;          // ngroups * d_state (b, c)
    int nheads;
    int t_inner;     // TESA heads * head size (q, k, v, o)
};

// Byte offsets of the layer's intermediates inside its workspace (256-byte aligned). The y region first
// holds the fp32 output of the joint B, C and dt projection (bcd: its weights side by side).
struct LayerLayout {
    size_t x, z, b, c, dt, q, k, v, y, o, bcd, core, blas, total;
};

constexpr size_t kGemmWorkspace = (size_t)64 << 20;  // reserved for hipBLASLt inside the layer's workspace

LayerLayout layer_layout(const LayerDims &d, size_t core_ws);

// Row-major D[M][Nout] = A[M][K] W[K][Nout] (+ D when accumulate) on hipBLASLt: bf16 A and W, fp32
// accumulation, D fp32 (d_f32) or bf16. Returns 0, or 1 with a message in msg.
int gemm_rowmajor(const void *A, const void *W, void *D, int64_t M, int64_t K, int64_t Nout, bool d_f32,
                  bool accumulate, void *ws, size_t ws_bytes, hipStream_t st, char *msg, size_t msg_len);

// The joint projection's rows [B | C | dt] (fp32, bc + bc + nheads wide) split into B and C (bf16) and
// dt = softplus(raw + bias) (fp32).
hipError_t layer_split_bcdt(const float *bcd, void *b, void *c, float *dt, const float *bias, int64_t tokens, int bc,
                            int nheads, hipStream_t st);
hipError_t layer_gated_norm(const void *y, void *z, const float *w, int64_t tokens, int channels, int groups,
                            float eps, hipStream_t st);

} // namespace mate
