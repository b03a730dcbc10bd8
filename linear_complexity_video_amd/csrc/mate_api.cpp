// C ABI of the MATE core: argument validation (before any launch), workspace
// sizing and kernel dispatch. See include/mate.h for the contract.
#include "mate.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>

#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

mate_status fail(mate_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

mate_status device_fail(hipError_t e, const char *what)
{
    return fail(MATE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxTokens = (int64_t)1 << 31;
// Launch grids carry heads, groups, review tokens and the batch on their y and z extents, which the device
// caps at 65536; larger counts are rejected here rather than failing at a launch.
constexpr int64_t kMaxGridYZ = 65535;

mate_status check_grid_yz(const char *what, int64_t v)
{
    if (v > kMaxGridYZ)
        return fail(MATE_ERR_UNSUPPORTED, "%s %lld above %lld is not built (launch grid extent)", what, (long long)v,
                    (long long)kMaxGridYZ);
    return MATE_OK;
}

mate_status check_grid(mate_grid g)
{
    if (g.batch <= 0 || g.T <= 0 || g.H <= 0 || g.W <= 0)
        return fail(MATE_ERR_SHAPE, "grid extents must be positive (batch=%lld T=%lld H=%lld W=%lld)",
                    (long long)g.batch, (long long)g.T, (long long)g.H, (long long)g.W);
    if (g.T > kMaxTokens || g.H > kMaxTokens || g.W > kMaxTokens ||
        g.T * g.H > kMaxTokens || g.T * g.H * g.W >= kMaxTokens || g.batch * g.T * g.H * g.W >= kMaxTokens)
        return fail(MATE_ERR_UNSUPPORTED, "grid too large: batch*T*H*W must stay below 2^31 tokens");
    return MATE_OK;
}

// Per-device one-time function attributes (LDS limits).
mate_status prepare_device()
{
    static std::atomic<int> done[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return MATE_OK;
    if (done[dev].load(std::memory_order_acquire)) return MATE_OK;
    if ((e = mate::ssd_portable_prepare()) != hipSuccess) return device_fail(e, "hipFuncSetAttribute");
    if ((e = mate::ssd_fast_prepare()) != hipSuccess) return device_fail(e, "hipFuncSetAttribute");
    if ((e = mate::ssd_backward_prepare()) != hipSuccess) return device_fail(e, "hipFuncSetAttribute");
    done[dev].store(1, std::memory_order_release);
    return MATE_OK;
}

bool valid_dtype(mate_dtype d) { return d == MATE_F32 || d == MATE_BF16; }
bool valid_algo(mate_algo a) { return a == MATE_ALGO_AUTO || a == MATE_ALGO_PORTABLE || a == MATE_ALGO_FAST; }

// Validates the SSD descriptor and fills the derived problem; `fast` tells
// which kernel family will run.
mate_status make_ssd_problem(mate_grid g, int order, const mate_ssd_desc *d, mate::SsdProblem &p, bool &fast)
{
    if (!d) return fail(MATE_ERR_NULL, "ssd descriptor is NULL");
    mate_status s = check_grid(g);
    if (s != MATE_OK) return s;
    if (order < 0 || order > MATE_ORDER_ZIGZAG) return fail(MATE_ERR_SHAPE, "order %d not in 0..4", order);
    if (d->nheads <= 0 || d->headdim <= 0 || d->d_state <= 0 || d->ngroups <= 0)
        return fail(MATE_ERR_SHAPE, "nheads, headdim, d_state and ngroups must be positive");
    if (d->chunk < 1) return fail(MATE_ERR_SHAPE, "chunk %d < 1", d->chunk);
    if (d->nheads % d->ngroups) return fail(MATE_ERR_SHAPE, "nheads %d not divisible by ngroups %d", d->nheads, d->ngroups);
    if (!valid_dtype(d->dtype)) return fail(MATE_ERR_SHAPE, "unknown dtype %d", (int)d->dtype);
    if (!valid_algo(d->algo)) return fail(MATE_ERR_SHAPE, "unknown algo %d", (int)d->algo);
    const bool pooled = d->pool_t || d->pool_h || d->pool_w;
    if (pooled) {
        if (d->pool_t <= 0 || d->pool_h <= 0 || d->pool_w <= 0)
            return fail(MATE_ERR_SHAPE, "pool extents must be all zero or all positive");
        if (g.T % d->pool_t || g.H % d->pool_h || g.W % d->pool_w)
            return fail(MATE_ERR_SHAPE, "pool %dx%dx%d does not divide the grid", d->pool_t, d->pool_h, d->pool_w);
    }
    if (d->headdim > 128 || d->d_state > 128)
        return fail(MATE_ERR_UNSUPPORTED, "headdim and d_state above 128 are not built");
    if (d->chunk > 128) return fail(MATE_ERR_UNSUPPORTED, "chunk above 128 is not built");
    if ((int64_t)d->nheads * g.batch * g.T * g.H * g.W >= kMaxTokens)
        return fail(MATE_ERR_UNSUPPORTED, "batch*tokens*nheads must stay below 2^31");
    p.batch = g.batch; p.T = g.T; p.H = g.H; p.W = g.W; p.N = g.T * g.H * g.W;
    p.nheads = d->nheads; p.headdim = d->headdim; p.d_state = d->d_state; p.ngroups = d->ngroups;
    p.chunk = d->chunk; p.order = order;
    p.pool_t = pooled ? d->pool_t : 0; p.pool_h = pooled ? d->pool_h : 0; p.pool_w = pooled ? d->pool_w : 0;
    p.R = pooled ? (g.T / d->pool_t) * (g.H / d->pool_h) * (g.W / d->pool_w) : 0;
    if ((s = check_grid_yz("batch", g.batch)) != MATE_OK || (s = check_grid_yz("nheads", d->nheads)) != MATE_OK ||
        (s = check_grid_yz("review tokens", p.R)) != MATE_OK)
        return s;
    if ((p.N + d->chunk - 1) / d->chunk > ((int64_t)1 << 22))
        return fail(MATE_ERR_UNSUPPORTED, "more than 2^22 chunks per sequence are not built (launch grid extent)");
    p.nch = (int)((p.N + d->chunk - 1) / d->chunk);
    p.nchR = (int)((p.R + d->chunk - 1) / d->chunk);
    p.dtype = d->dtype == MATE_BF16 ? 1 : 0;
    const bool has_fast = mate::ssd_fast_supports(p);
    if (d->algo == MATE_ALGO_FAST && !has_fast)
        return fail(MATE_ERR_UNSUPPORTED, "no MFMA scan kernel for dtype %d headdim %d d_state %d chunk %d",
                    (int)d->dtype, d->headdim, d->d_state, d->chunk);
    fast = d->algo != MATE_ALGO_PORTABLE && has_fast;
    return MATE_OK;
}

// Validates the Mamba (selective scan) descriptor and fills the derived problem.
mate_status make_mamba_problem(mate_grid g, int order, const mate_mamba_desc *d, mate::MambaProblem &p)
{
    if (!d) return fail(MATE_ERR_NULL, "mamba descriptor is NULL");
    mate_status s = check_grid(g);
    if (s != MATE_OK) return s;
    if (order < 0 || order > MATE_ORDER_ZIGZAG) return fail(MATE_ERR_SHAPE, "order %d not in 0..4", order);
    if (d->channels <= 0 || d->d_state <= 0) return fail(MATE_ERR_SHAPE, "channels and d_state must be positive");
    if (!valid_dtype(d->dtype)) return fail(MATE_ERR_SHAPE, "unknown dtype %d", (int)d->dtype);
    const bool pooled = d->pool_t || d->pool_h || d->pool_w;
    if (pooled) {
        if (d->pool_t <= 0 || d->pool_h <= 0 || d->pool_w <= 0)
            return fail(MATE_ERR_SHAPE, "pool extents must be all zero or all positive");
        if (g.T % d->pool_t || g.H % d->pool_h || g.W % d->pool_w)
            return fail(MATE_ERR_SHAPE, "pool %dx%dx%d does not divide the grid", d->pool_t, d->pool_h, d->pool_w);
    }
    if (d->d_state != 8 && d->d_state != 16 && d->d_state != 32)
        return fail(MATE_ERR_UNSUPPORTED, "d_state %d not built (8, 16 or 32)", d->d_state);
    if ((int64_t)d->channels * g.batch * g.T * g.H * g.W >= ((int64_t)1 << 40))
        return fail(MATE_ERR_UNSUPPORTED, "batch*tokens*channels must stay below 2^40");
    if (d->channels > (1 << 26))
        return fail(MATE_ERR_UNSUPPORTED, "more than 2^26 channels are not built (launch grid extent)");
    p.batch = g.batch; p.T = g.T; p.H = g.H; p.W = g.W;
    p.channels = d->channels; p.d_state = d->d_state; p.order = order;
    p.pool_t = pooled ? d->pool_t : 0; p.pool_h = pooled ? d->pool_h : 0; p.pool_w = pooled ? d->pool_w : 0;
    p.R = pooled ? (g.T / d->pool_t) * (g.H / d->pool_h) * (g.W / d->pool_w) : 0;
    if ((s = check_grid_yz("batch", g.batch)) != MATE_OK || (s = check_grid_yz("review tokens", p.R)) != MATE_OK)
        return s;
    p.dtype = d->dtype == MATE_BF16 ? 1 : 0;
    return MATE_OK;
}

mate_status make_tesa_problem(mate_grid g, const mate_tesa_desc *d, mate::TesaProblem &p, bool &fast)
{
    if (!d) return fail(MATE_ERR_NULL, "tesa descriptor is NULL");
    mate_status s = check_grid(g);
    if (s != MATE_OK) return s;
    if (d->nheads <= 0 || d->headdim <= 0) return fail(MATE_ERR_SHAPE, "nheads and headdim must be positive");
    if (d->win_t <= 0 || d->win_h <= 0 || d->win_w <= 0) return fail(MATE_ERR_SHAPE, "window extents must be positive");
    if (g.T % d->win_t || g.H % d->win_h || g.W % d->win_w)
        return fail(MATE_ERR_SHAPE, "window %dx%dx%d does not divide the grid", d->win_t, d->win_h, d->win_w);
    if (d->shift_t < 0 || d->shift_t >= d->win_t || d->shift_h < 0 || d->shift_h >= d->win_h || d->shift_w < 0 ||
        d->shift_w >= d->win_w)
        return fail(MATE_ERR_SHAPE, "shift (%d,%d,%d) outside [0, window)", d->shift_t, d->shift_h, d->shift_w);
    if (!valid_dtype(d->dtype)) return fail(MATE_ERR_SHAPE, "unknown dtype %d", (int)d->dtype);
    if (!valid_algo(d->algo)) return fail(MATE_ERR_SHAPE, "unknown algo %d", (int)d->algo);
    if ((int64_t)d->nheads * g.batch * g.T * g.H * g.W >= kMaxTokens)
        return fail(MATE_ERR_UNSUPPORTED, "batch*tokens*nheads must stay below 2^31");
    if ((s = check_grid_yz("batch", g.batch)) != MATE_OK || (s = check_grid_yz("nheads", d->nheads)) != MATE_OK)
        return s;
    p.batch = g.batch; p.T = g.T; p.H = g.H; p.W = g.W;
    p.nheads = d->nheads; p.headdim = d->headdim;
    p.wt = d->win_t; p.wh = d->win_h; p.ww = d->win_w;
    p.st = d->shift_t; p.sh = d->shift_h; p.sw = d->shift_w;
    p.nrt = (int)(g.T / d->win_t) + (d->shift_t ? 1 : 0);
    p.nrh = (int)(g.H / d->win_h) + (d->shift_h ? 1 : 0);
    p.nrw = (int)(g.W / d->win_w) + (d->shift_w ? 1 : 0);
    if ((int64_t)p.nrt * p.nrh * p.nrw > ((int64_t)1 << 22))
        return fail(MATE_ERR_UNSUPPORTED, "more than 2^22 window regions are not built (launch grid extent)");
    p.scale = d->scale;
    p.dtype = d->dtype == MATE_BF16 ? 1 : 0;
    const bool has_fast = mate::tesa_fast_supports(p);
    const bool has_portable = mate::tesa_portable_supports(p);
    if (d->algo == MATE_ALGO_FAST && !has_fast)
        return fail(MATE_ERR_UNSUPPORTED, "no MFMA TESA kernel for dtype %d headdim %d", (int)d->dtype, d->headdim);
    if (d->algo == MATE_ALGO_PORTABLE && !has_portable)
        return fail(MATE_ERR_UNSUPPORTED, "portable TESA needs headdim in {8,16,32,64,128} and <= 1024-token windows");
    if (!has_fast && !has_portable)
        return fail(MATE_ERR_UNSUPPORTED, "TESA not built for headdim %d with %dx%dx%d windows", d->headdim, d->win_t,
                    d->win_h, d->win_w);
    fast = d->algo != MATE_ALGO_PORTABLE && has_fast;
    return MATE_OK;
}

size_t ssd_workspace(const mate::SsdProblem &p, bool fast)
{
    return fast ? mate::ssd_fast_workspace(p) : mate::ssd_portable_workspace(p);
}

mate_status check_ssd_tensors(const mate_ssd_tensors *t)
{
    if (!t) return fail(MATE_ERR_NULL, "ssd tensors struct is NULL");
    if (!t->x || !t->b || !t->c || !t->dt || !t->a || !t->d || !t->y)
        return fail(MATE_ERR_NULL, "an ssd tensor pointer (x, b, c, dt, a, d, y) is NULL");
    if (((uintptr_t)t->x | (uintptr_t)t->b | (uintptr_t)t->c | (uintptr_t)t->y) & 15)
        return fail(MATE_ERR_UNSUPPORTED, "x, b, c and y must be 16-byte aligned");
    if (((uintptr_t)t->dt | (uintptr_t)t->a | (uintptr_t)t->d) & 3)
        return fail(MATE_ERR_UNSUPPORTED, "dt, a and d must be 4-byte aligned");
    return MATE_OK;
}

mate_status check_tesa_tensors(const mate_tesa_tensors *t)
{
    if (!t) return fail(MATE_ERR_NULL, "tesa tensors struct is NULL");
    if (!t->q || !t->k || !t->v || !t->o) return fail(MATE_ERR_NULL, "a tesa tensor pointer (q, k, v, o) is NULL");
    if (((uintptr_t)t->q | (uintptr_t)t->k | (uintptr_t)t->v | (uintptr_t)t->o) & 15)
        return fail(MATE_ERR_UNSUPPORTED, "q, k, v and o must be 16-byte aligned");
    return MATE_OK;
}

} // namespace

extern "C" {

int mate_abi_version(void) { return MATE_ABI_VERSION; }

const char *mate_status_string(mate_status s)
{
    switch (s) {
    case MATE_OK: return "MATE_OK";
    case MATE_ERR_NULL: return "MATE_ERR_NULL: a required pointer is NULL";
    case MATE_ERR_SHAPE: return "MATE_ERR_SHAPE: invalid extents, order, window, shift, pool or chunk";
    case MATE_ERR_UNSUPPORTED: return "MATE_ERR_UNSUPPORTED: valid for the method but not built";
    case MATE_ERR_WORKSPACE: return "MATE_ERR_WORKSPACE: workspace missing or too small";
    case MATE_ERR_DEVICE: return "MATE_ERR_DEVICE: a HIP call or kernel launch failed";
    }
    return "unknown mate_status";
}

const char *mate_last_error(void) { return g_err; }

mate_status mate_rms_reorder(const void *src, void *dst, mate_grid g, int64_t row_bytes, int order, int flip,
                             int inverse, void *stream)
{
    if (!src || !dst) return fail(MATE_ERR_NULL, "src or dst is NULL");
    mate_status s = check_grid(g);
    if (s != MATE_OK) return s;
    if (row_bytes <= 0) return fail(MATE_ERR_SHAPE, "row_bytes %lld must be positive", (long long)row_bytes);
    if (order < 0 || order > MATE_ORDER_ZIGZAG) return fail(MATE_ERR_SHAPE, "order %d not in 0..4", order);
    const int64_t rows = g.batch * g.T * g.H * g.W;
    if (row_bytes > ((int64_t)1 << 40) / rows) return fail(MATE_ERR_UNSUPPORTED, "tensor above 1 TiB");
    // the kernels count a row's vectors in 32 bits
    if (row_bytes >= ((int64_t)1 << 32) - 1024)
        return fail(MATE_ERR_UNSUPPORTED, "rows of 4 GiB or more are not built");
    const uintptr_t bytes = (uintptr_t)(rows * row_bytes);
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (a < b + bytes && b < a + bytes) return fail(MATE_ERR_SHAPE, "src and dst overlap");
    hipError_t e = mate::launch_rms_reorder(src, dst, g.batch, g.T, g.H, g.W, row_bytes, order, flip ? 1 : 0,
                                            inverse ? 1 : 0, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "rms reorder launch");
    return MATE_OK;
}

size_t mate_bissd_workspace_size(mate_grid g, const mate_ssd_desc *d)
{
    mate::SsdProblem p;
    bool fast = false;
    if (make_ssd_problem(g, 0, d, p, fast) != MATE_OK) return 0;
    return ssd_workspace(p, fast);
}

mate_status mate_bissd_scan(const mate_ssd_tensors *t, mate_grid g, int order, const mate_ssd_desc *d,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    mate_status s = check_ssd_tensors(t);
    if (s != MATE_OK) return s;
    mate::SsdProblem p;
    bool fast = false;
    if ((s = make_ssd_problem(g, order, d, p, fast)) != MATE_OK) return s;
    const size_t need = ssd_workspace(p, fast);
    if (!workspace || workspace_bytes < need)
        return fail(MATE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);
    if ((uintptr_t)workspace & 255) return fail(MATE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if ((s = prepare_device()) != MATE_OK) return s;
    mate::SsdArgs a{t->x, t->b, t->c, t->dt, t->a, t->d, t->y};
    hipError_t e = fast ? mate::ssd_fast(p, a, workspace, (hipStream_t)stream)
                        : mate::ssd_portable(p, a, workspace, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "bissd launch");
    return MATE_OK;
}

mate_status mate_bissd_scan_noalloc(const mate_ssd_tensors *t, mate_grid g, int order, const mate_ssd_desc *d,
                                    void *stream)
{
    mate_status s = check_ssd_tensors(t);
    if (s != MATE_OK) return s;
    mate::SsdProblem p;
    bool fast = false;
    if ((s = make_ssd_problem(g, order, d, p, fast)) != MATE_OK) return s;
    const size_t need = ssd_workspace(p, fast);
    if (need > MATE_STATIC_SCRATCH_BYTES)
        return fail(MATE_ERR_WORKSPACE, "the scan needs %zu bytes of scratch; the library's static scratch holds %zu",
                    need, (size_t)MATE_STATIC_SCRATCH_BYTES);
    if ((s = prepare_device()) != MATE_OK) return s;
    void *ws = nullptr;
    hipError_t e = mate::static_scratch(&ws);
    if (e != hipSuccess) return device_fail(e, "static scratch address");
    mate::SsdArgs a{t->x, t->b, t->c, t->dt, t->a, t->d, t->y};
    e = fast ? mate::ssd_fast(p, a, ws, (hipStream_t)stream) : mate::ssd_portable(p, a, ws, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "bissd launch");
    return MATE_OK;
}

size_t mate_bissd_backward_workspace_size(mate_grid g, const mate_ssd_desc *d)
{
    mate::SsdProblem p;
    bool fast = false;
    if (make_ssd_problem(g, 0, d, p, fast) != MATE_OK || !mate::ssd_backward_supports(p)) return 0;
    return mate::ssd_backward_workspace(p);
}

mate_status mate_bissd_backward(const mate_ssd_grad_tensors *t, mate_grid g, int order, const mate_ssd_desc *d,
                                void *workspace, size_t workspace_bytes, void *stream)
{
    if (!t) return fail(MATE_ERR_NULL, "ssd gradient tensors struct is NULL");
    if (!t->x || !t->b || !t->c || !t->dt || !t->a || !t->d || !t->dy || !t->dx || !t->db || !t->dc || !t->ddt ||
        !t->da || !t->dd)
        return fail(MATE_ERR_NULL, "an ssd gradient tensor pointer is NULL");
    if (((uintptr_t)t->x | (uintptr_t)t->b | (uintptr_t)t->c | (uintptr_t)t->dy | (uintptr_t)t->dx |
         (uintptr_t)t->db | (uintptr_t)t->dc) & 15)
        return fail(MATE_ERR_UNSUPPORTED, "x, b, c, dy, dx, db and dc must be 16-byte aligned");
    if (((uintptr_t)t->dt | (uintptr_t)t->a | (uintptr_t)t->d | (uintptr_t)t->ddt | (uintptr_t)t->da |
         (uintptr_t)t->dd) & 3)
        return fail(MATE_ERR_UNSUPPORTED, "dt, a, d, ddt, da and dd must be 4-byte aligned");
    mate::SsdProblem p;
    bool fast = false;
    mate_status s = make_ssd_problem(g, order, d, p, fast);
    if (s != MATE_OK) return s;
    if (!mate::ssd_backward_supports(p))
        return fail(MATE_ERR_UNSUPPORTED, "the scan's backward is built for headdim 16, 32 or 64, d_state <= 128 "
                                          "(a multiple of 8) and ceil(review tokens / 16) * batch * nheads < 2^24");
    const size_t need = mate::ssd_backward_workspace(p);
    if (!workspace || workspace_bytes < need)
        return fail(MATE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);
    if ((uintptr_t)workspace & 255) return fail(MATE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if ((s = prepare_device()) != MATE_OK) return s;
    mate::SsdGradArgs a{t->x, t->b, t->c, t->dt, t->a, t->d, t->dy, t->dx, t->db, t->dc, t->ddt, t->da, t->dd};
    hipError_t e = mate::ssd_backward(p, a, workspace, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "bissd backward launch");
    return MATE_OK;
}

size_t mate_bimamba_workspace_size(mate_grid g, const mate_mamba_desc *d)
{
    mate::MambaProblem p;
    if (make_mamba_problem(g, 0, d, p) != MATE_OK) return 0;
    return mate::mamba_workspace(p);
}

mate_status mate_bimamba_scan(const mate_ssd_tensors *t, mate_grid g, int order, const mate_mamba_desc *d,
                              void *workspace, size_t workspace_bytes, void *stream)
{
    mate_status s = check_ssd_tensors(t);
    if (s != MATE_OK) return s;
    mate::MambaProblem p;
    if ((s = make_mamba_problem(g, order, d, p)) != MATE_OK) return s;
    const size_t need = mate::mamba_workspace(p);
    if (!workspace || workspace_bytes < need)
        return fail(MATE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);
    if ((uintptr_t)workspace & 255) return fail(MATE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    mate::MambaArgs a{t->x, t->b, t->c, t->dt, t->a, t->d, t->y};
    hipError_t e = mate::mamba_scan(p, a, workspace, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "bimamba launch");
    return MATE_OK;
}

mate_status mate_tesa(const mate_tesa_tensors *t, mate_grid g, const mate_tesa_desc *d, void *stream)
{
    mate_status s = check_tesa_tensors(t);
    if (s != MATE_OK) return s;
    mate::TesaProblem p;
    bool fast = false;
    if ((s = make_tesa_problem(g, d, p, fast)) != MATE_OK) return s;
    if ((s = prepare_device()) != MATE_OK) return s;
    mate::TesaArgs a{t->q, t->k, t->v, t->o};
    hipError_t e = fast ? mate::tesa_fast(p, a, (hipStream_t)stream) : mate::tesa_portable(p, a, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "tesa launch");
    return MATE_OK;
}

size_t mate_tesa_backward_workspace_size(mate_grid g, const mate_tesa_desc *d)
{
    mate::TesaProblem p;
    bool fast = false;
    if (make_tesa_problem(g, d, p, fast) != MATE_OK || !mate::tesa_backward_supports(p)) return 0;
    return mate::tesa_backward_workspace(p);
}

mate_status mate_tesa_backward(const mate_tesa_grad_tensors *t, mate_grid g, const mate_tesa_desc *d,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (!t) return fail(MATE_ERR_NULL, "tesa gradient tensors struct is NULL");
    if (!t->q || !t->k || !t->v || !t->dout || !t->dq || !t->dk || !t->dv)
        return fail(MATE_ERR_NULL, "a tesa gradient tensor pointer (q, k, v, dout, dq, dk, dv) is NULL");
    if (((uintptr_t)t->q | (uintptr_t)t->k | (uintptr_t)t->v | (uintptr_t)t->dout | (uintptr_t)t->dq |
         (uintptr_t)t->dk | (uintptr_t)t->dv) & 15)
        return fail(MATE_ERR_UNSUPPORTED, "q, k, v, dout, dq, dk and dv must be 16-byte aligned");
    mate::TesaProblem p;
    bool fast = false;
    mate_status s = make_tesa_problem(g, d, p, fast);
    if (s != MATE_OK) return s;
    if (!mate::tesa_backward_supports(p))
        return fail(MATE_ERR_UNSUPPORTED, "tesa backward is built for bf16, headdim 64 or 128, windows of at most 4096 tokens");
    const size_t need = mate::tesa_backward_workspace(p);
    if (!workspace || workspace_bytes < need)
        return fail(MATE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);
    if ((uintptr_t)workspace & 255) return fail(MATE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    mate::TesaGradArgs a{t->q, t->k, t->v, t->dout, t->dq, t->dk, t->dv};
    hipError_t e = mate::tesa_backward(p, a, workspace, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "tesa backward launch");
    return MATE_OK;
}

size_t mate_forward_workspace_size(mate_grid g, const mate_ssd_desc *sd, const mate_tesa_desc *td)
{
    mate::TesaProblem tp;
    bool tf = false;
    if (make_tesa_problem(g, td, tp, tf) != MATE_OK) return 0;
    return mate_bissd_workspace_size(g, sd);
}

mate_status mate_forward(const mate_ssd_tensors *s, const mate_ssd_desc *sd, const mate_tesa_tensors *a,
                         const mate_tesa_desc *td, mate_grid g, int order, void *workspace, size_t workspace_bytes,
                         void *stream)
{
    // Validate everything before the first launch so that a rejected call writes nothing.
    mate_status st = check_ssd_tensors(s);
    if (st != MATE_OK) return st;
    if ((st = check_tesa_tensors(a)) != MATE_OK) return st;
    mate::SsdProblem sp;
    mate::TesaProblem tp;
    bool sfast = false, tfast = false;
    if ((st = make_ssd_problem(g, order, sd, sp, sfast)) != MATE_OK) return st;
    if ((st = make_tesa_problem(g, td, tp, tfast)) != MATE_OK) return st;
    const size_t need = ssd_workspace(sp, sfast);
    if (!workspace || workspace_bytes < need)
        return fail(MATE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);
    if ((uintptr_t)workspace & 255) return fail(MATE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if ((st = prepare_device()) != MATE_OK) return st;
    // Both branches run on the caller's stream, one after the other: the TE branch's persistent
    // workgroups hold every CU, so running it beside the scan on a second stream overlaps little, and
    // one stream keeps the call free of library-owned streams and events.
    const hipStream_t stream_h = (hipStream_t)stream;
    mate::SsdArgs sa{s->x, s->b, s->c, s->dt, s->a, s->d, s->y};
    mate::TesaArgs ta{a->q, a->k, a->v, a->o};
    hipError_t e = tfast ? mate::tesa_fast(tp, ta, stream_h) : mate::tesa_portable(tp, ta, stream_h);
    if (e != hipSuccess) return device_fail(e, "forward: tesa launch");
    e = sfast ? mate::ssd_fast(sp, sa, workspace, stream_h) : mate::ssd_portable(sp, sa, workspace, stream_h);
    if (e != hipSuccess) return device_fail(e, "forward: bissd launch");
    return MATE_OK;
}

} // extern "C"

namespace {

// Validates a layer call's descriptors (everything but the pointers); fills the branch problems and the
// layer's dimensions.
mate_status make_layer(mate_grid g, int order, const mate_layer_desc *ld, const mate_ssd_desc *sd,
                       const mate_tesa_desc *td, mate::SsdProblem &sp, bool &sfast, mate::TesaProblem &tp,
                       bool &tfast, mate::LayerDims &dims)
{
    if (!ld) return fail(MATE_ERR_NULL, "layer descriptor is NULL");
    mate_status st = make_ssd_problem(g, order, sd, sp, sfast);
    if (st != MATE_OK) return st;
    if ((st = make_tesa_problem(g, td, tp, tfast)) != MATE_OK) return st;
    if (sd->dtype != MATE_BF16 || td->dtype != MATE_BF16)
        return fail(MATE_ERR_UNSUPPORTED, "mate_layer runs in bf16 (both descriptors' dtype)");
    if (ld->d_model <= 0 || ld->d_model % 8)
        return fail(MATE_ERR_SHAPE, "d_model %d must be a positive multiple of 8", ld->d_model);
    if (!(ld->norm_eps >= 0.f)) return fail(MATE_ERR_SHAPE, "norm_eps must be >= 0");
    const int inner = sd->nheads * sd->headdim;
    if (sd->ngroups > 64 || (inner / sd->ngroups) % 8)
        return fail(MATE_ERR_UNSUPPORTED, "the gated norm needs ngroups <= 64 and nheads*headdim/ngroups a multiple of 8");
    dims.tokens = g.batch * g.T * g.H * g.W;
    dims.d_model = ld->d_model;
    dims.inner = inner;
    dims.bc = sd->ngroups * sd->d_state;
    dims.nheads = sd->nheads;
    dims.t_inner = td->nheads * td->headdim;
    if ((int64_t)dims.tokens * std::max({dims.d_model, dims.inner, dims.t_inner}) >= ((int64_t)1 << 40))
        return fail(MATE_ERR_UNSUPPORTED, "layer too large");
    return MATE_OK;
}

} // namespace

extern "C" {

size_t mate_layer_workspace_size(mate_grid g, const mate_layer_desc *ld, const mate_ssd_desc *sd,
                                 const mate_tesa_desc *td)
{
    mate::SsdProblem sp;
    mate::TesaProblem tp;
    mate::LayerDims dims;
    bool sfast = false, tfast = false;
    if (make_layer(g, 0, ld, sd, td, sp, sfast, tp, tfast, dims) != MATE_OK) return 0;
    return mate::layer_layout(dims, ssd_workspace(sp, sfast)).total;
}

mate_status mate_layer(const void *h, void *out, const mate_layer_weights *w, const mate_layer_desc *ld,
                       const mate_ssd_desc *sd, const mate_tesa_desc *td, mate_grid g, int order, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    if (!h || !out) return fail(MATE_ERR_NULL, "h or out is NULL");
    if (!w) return fail(MATE_ERR_NULL, "layer weights struct is NULL");
    if (!w->w_x || !w->w_z || !w->w_b || !w->w_c || !w->w_dt || !w->w_ma_out || !w->dt_bias || !w->a || !w->d ||
        !w->norm_w || !w->w_q || !w->w_k || !w->w_v || !w->w_te_out)
        return fail(MATE_ERR_NULL, "a layer weight pointer is NULL");
    if (((uintptr_t)h | (uintptr_t)out) & 15) return fail(MATE_ERR_UNSUPPORTED, "h and out must be 16-byte aligned");
    if (((uintptr_t)w->w_x | (uintptr_t)w->w_z | (uintptr_t)w->w_b | (uintptr_t)w->w_c | (uintptr_t)w->w_dt |
         (uintptr_t)w->w_ma_out | (uintptr_t)w->w_q | (uintptr_t)w->w_k | (uintptr_t)w->w_v |
         (uintptr_t)w->w_te_out) & 15)
        return fail(MATE_ERR_UNSUPPORTED, "weight matrices must be 16-byte aligned");
    if (((uintptr_t)w->dt_bias | (uintptr_t)w->a | (uintptr_t)w->d | (uintptr_t)w->norm_w) & 3)
        return fail(MATE_ERR_UNSUPPORTED, "dt_bias, a, d and norm_w must be 4-byte aligned");
    mate::SsdProblem sp;
    mate::TesaProblem tp;
    mate::LayerDims dims;
    bool sfast = false, tfast = false;
    mate_status st = make_layer(g, order, ld, sd, td, sp, sfast, tp, tfast, dims);
    if (st != MATE_OK) return st;
    const mate::LayerLayout l = mate::layer_layout(dims, ssd_workspace(sp, sfast));
    if (!workspace || workspace_bytes < l.total)
        return fail(MATE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                    l.total);
    if ((uintptr_t)workspace & 255) return fail(MATE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if ((st = prepare_device()) != MATE_OK) return st;

    const hipStream_t sh = (hipStream_t)stream;
    char *ws = (char *)workspace;
    void *x = ws + l.x, *z = ws + l.z, *b = ws + l.b, *c = ws + l.c, *q = ws + l.q, *k = ws + l.k, *v = ws + l.v;
    void *y = ws + l.y, *o = ws + l.o, *blas = ws + l.blas;
    float *dt = (float *)(ws + l.dt);
    const int64_t M = dims.tokens, K = dims.d_model;
    char msg[256];
    struct Proj {
        const void *wm;
        void *dst;
        int64_t n;
        bool f32;
    };
    const Proj ins[] = {{w->w_x, x, dims.inner, false},       {w->w_z, z, dims.inner, false},
                        {w->w_q, q, dims.t_inner, false},     {w->w_k, k, dims.t_inner, false},
                        {w->w_v, v, dims.t_inner, false}};
    for (const Proj &pj : ins)
        if (mate::gemm_rowmajor(h, pj.wm, pj.dst, M, K, pj.n, pj.f32, false, blas, mate::kGemmWorkspace, sh, msg,
                                sizeof(msg)))
            return fail(MATE_ERR_DEVICE, "layer in-projection: %s", msg);
    // B, C and dt from one GEMM over their weights side by side (the narrow projections read h once), its
    // fp32 rows in the y region (free until the scan), then split.
    {
        const size_t nb = (size_t)2 * dims.bc + dims.nheads, e2 = 2;
        char *wb = ws + l.bcd;
        hipError_t e = hipMemcpy2DAsync(wb, nb * e2, w->w_b, dims.bc * e2, dims.bc * e2, K, hipMemcpyDeviceToDevice, sh);
        if (e == hipSuccess)
            e = hipMemcpy2DAsync(wb + dims.bc * e2, nb * e2, w->w_c, dims.bc * e2, dims.bc * e2, K,
                                 hipMemcpyDeviceToDevice, sh);
        if (e == hipSuccess)
            e = hipMemcpy2DAsync(wb + 2 * dims.bc * e2, nb * e2, w->w_dt, dims.nheads * e2, dims.nheads * e2, K,
                                 hipMemcpyDeviceToDevice, sh);
        if (e != hipSuccess) return device_fail(e, "layer: joint projection weights");
        if (mate::gemm_rowmajor(h, wb, y, M, K, (int64_t)nb, true, false, blas, mate::kGemmWorkspace, sh, msg,
                                sizeof(msg)))
            return fail(MATE_ERR_DEVICE, "layer in-projection (B, C, dt): %s", msg);
        e = mate::layer_split_bcdt((const float *)y, b, c, dt, w->dt_bias, M, dims.bc, dims.nheads, sh);
        if (e != hipSuccess) return device_fail(e, "layer: B, C and dt");
    }
    hipError_t e;
    const mate::TesaArgs ta{q, k, v, o};
    e = tfast ? mate::tesa_fast(tp, ta, sh) : mate::tesa_portable(tp, ta, sh);
    if (e != hipSuccess) return device_fail(e, "layer: tesa launch");
    const mate::SsdArgs sa{x, b, c, dt, w->a, w->d, y};
    e = sfast ? mate::ssd_fast(sp, sa, ws + l.core, sh) : mate::ssd_portable(sp, sa, ws + l.core, sh);
    if (e != hipSuccess) return device_fail(e, "layer: bissd launch");
    e = mate::layer_gated_norm(y, z, w->norm_w, M, dims.inner, sd->ngroups, ld->norm_eps, sh);
    if (e != hipSuccess) return device_fail(e, "layer: gated norm");
    if (mate::gemm_rowmajor(z, w->w_ma_out, out, M, dims.inner, K, false, false, blas, mate::kGemmWorkspace, sh,
                            msg, sizeof(msg)) ||
        mate::gemm_rowmajor(o, w->w_te_out, out, M, dims.t_inner, K, false, true, blas, mate::kGemmWorkspace, sh,
                            msg, sizeof(msg)))
        return fail(MATE_ERR_DEVICE, "layer out-projection: %s", msg);
    return MATE_OK;
}

} // extern "C"
