// One MATE layer around the core: the in- and out-projection GEMMs on
// hipBLASLt, the workspace layout of the layer's intermediates, and the
// sequence of launches. Validation happens in mate_api.cpp before any of this
// runs.
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>

#include "launch.hpp"

namespace mate {

namespace {

constexpr int kMaxDevices = 64;

struct GemmKey {
    int dev;
    int64_t M, K, Nout;
    bool d_f32, accumulate;
    bool operator<(const GemmKey &o) const
    {
        return std::tie(dev, M, K, Nout, d_f32, accumulate) < std::tie(o.dev, o.M, o.K, o.Nout, o.d_f32, o.accumulate);
    }
};

struct GemmPlan {
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
};

std::mutex g_mu;                      // guards the handles and the plan cache
std::mutex g_call_mu[kMaxDevices];    // one enqueue at a time per device's handle
hipblasLtHandle_t g_handle[kMaxDevices] = {};
std::map<GemmKey, GemmPlan> g_plans;

const char *blas_name(hipblasStatus_t s)
{
    switch (s) {
    case HIPBLAS_STATUS_SUCCESS: return "success";
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "not initialized";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "allocation failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "invalid value";
    case HIPBLAS_STATUS_MAPPING_ERROR: return "mapping error";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "execution failed";
    case HIPBLAS_STATUS_INTERNAL_ERROR: return "internal error";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "not supported";
    default: return "error";
    }
}

// The plan of one GEMM shape on the current device (created on first use, kept for the process); the
// hipBLASLt handle of the device likewise. Called with g_mu held.
int plan_for(const GemmKey &key, GemmPlan **out, char *msg, size_t msg_len)
{
    auto it = g_plans.find(key);
    if (it != g_plans.end()) {
        *out = &it->second;
        return 0;
    }
    hipblasStatus_t s;
    if (!g_handle[key.dev] && (s = hipblasLtCreate(&g_handle[key.dev])) != HIPBLAS_STATUS_SUCCESS) {
        snprintf(msg, msg_len, "hipblasLtCreate: %s", blas_name(s));
        return 1;
    }
    // Row-major D[M][Nout] = A[M][K] W[K][Nout] is the column-major product D^T = W^T A^T, with W^T the
    // column-major Nout x K matrix stored as W and A^T the column-major K x M matrix stored as A.
    GemmPlan p;
    auto release = [&]() {
        if (p.op) hipblasLtMatmulDescDestroy(p.op);
        if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
        if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
        if (p.d) hipblasLtMatrixLayoutDestroy(p.d);
    };
    const hipDataType dt = key.d_f32 ? HIP_R_32F : HIP_R_16BF;
    if ((s = hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F)) != HIPBLAS_STATUS_SUCCESS ||
        (s = hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, key.Nout, key.K, key.Nout)) != HIPBLAS_STATUS_SUCCESS ||
        (s = hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, key.K, key.M, key.K)) != HIPBLAS_STATUS_SUCCESS ||
        (s = hipblasLtMatrixLayoutCreate(&p.d, dt, key.Nout, key.M, key.Nout)) != HIPBLAS_STATUS_SUCCESS) {
        release();
        snprintf(msg, msg_len, "hipBLASLt descriptors: %s", blas_name(s));
        return 1;
    }
    hipblasLtMatmulPreference_t pref = nullptr;
    uint64_t ws_max = kGemmWorkspace;
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    if ((s = hipblasLtMatmulPreferenceCreate(&pref)) != HIPBLAS_STATUS_SUCCESS ||
        (s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws_max,
                                                   sizeof(ws_max))) != HIPBLAS_STATUS_SUCCESS ||
        (s = hipblasLtMatmulAlgoGetHeuristic(g_handle[key.dev], p.op, p.a, p.b, p.d, p.d, pref, 1, res, &found)) !=
            HIPBLAS_STATUS_SUCCESS ||
        found < 1) {
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
        release();
        snprintf(msg, msg_len, "hipBLASLt has no algorithm for %lld x %lld x %lld (%s)", (long long)key.M,
                 (long long)key.K, (long long)key.Nout, found < 1 ? "none found" : blas_name(s));
        return 1;
    }
    hipblasLtMatmulPreferenceDestroy(pref);
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    *out = &(g_plans[key] = p);
    return 0;
}

} // namespace

int gemm_rowmajor(const void *A, const void *Wt, void *D, int64_t M, int64_t K, int64_t Nout, bool d_f32,
                  bool accumulate, void *ws, size_t ws_bytes, hipStream_t st, char *msg, size_t msg_len)
{
    if (M == 0) return 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        snprintf(msg, msg_len, "hipGetDevice: %s", hipGetErrorString(e));
        return 1;
    }
    GemmPlan *p = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (plan_for(GemmKey{dev, M, K, Nout, d_f32, accumulate}, &p, msg, msg_len)) return 1;
    }
    if (p->ws > ws_bytes) {
        snprintf(msg, msg_len, "GEMM workspace of %zu bytes needed, %zu reserved", p->ws, ws_bytes);
        return 1;
    }
    const float alpha = 1.f, beta = accumulate ? 1.f : 0.f;
    hipblasStatus_t s;
    {
        std::lock_guard<std::mutex> lk(g_call_mu[dev]);
        s = hipblasLtMatmul(g_handle[dev], p->op, &alpha, Wt, p->a, A, p->b, &beta, D, p->d, D, p->d, &p->algo, ws,
                            p->ws, st);
    }
    if (s != HIPBLAS_STATUS_SUCCESS) {
        snprintf(msg, msg_len, "hipblasLtMatmul %lld x %lld x %lld: %s", (long long)M, (long long)K,
                 (long long)Nout, blas_name(s));
        return 1;
    }
    return 0;
}

LayerLayout layer_layout(const LayerDims &d, size_t core_ws)
{
    LayerLayout l{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (off + bytes + 255) & ~(size_t)255;
        return o;
    };
    const size_t n = (size_t)d.tokens;
    l.x = take(n * d.inner * 2);
    l.z = take(n * d.inner * 2);
    l.b = take(n * d.bc * 2);
    l.c = take(n * d.bc * 2);
    l.dt = take(n * d.nheads * 4);
    l.q = take(n * d.t_inner * 2);
    l.k = take(n * d.t_inner * 2);
    l.v = take(n * d.t_inner * 2);
    const size_t nbcd = (size_t)2 * d.bc + d.nheads;  // joint projection width
    l.y = take(std::max(n * d.inner * 2, n * nbcd * 4));
    l.o = take(n * d.t_inner * 2);
    l.bcd = take((size_t)d.d_model * nbcd * 2);
    l.core = take(core_ws);
    l.blas = take(kGemmWorkspace);
    l.total = off;
    return l;
}

} // namespace mate
