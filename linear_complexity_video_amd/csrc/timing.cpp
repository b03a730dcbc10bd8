// HIP event pairs around the launches of one armed kernel, summed on request.
#include "timing.hpp"

#include <cstring>
#include <mutex>
#include <vector>

#include "mate.h"

namespace mate {
namespace timing {

std::atomic<int> armed{-1};

namespace {

struct Pair {
    hipEvent_t begin = nullptr, end = nullptr;
};

std::mutex g_mu;
std::vector<Pair> g_pairs;   // created on demand, reused across timings
size_t g_used = 0;           // pairs holding a recorded launch
bool g_open = false;         // a begin is recorded without its end
hipError_t g_error = hipSuccess;

const char *const kNames[K_COUNT] = {"rms_reorder", "ssd_pool", "ssd_prep", "ssd_cb",
                                     "ssd_states", "ssd_seg_pass", "ssd_out", "tesa", "mamba_scan",
                                     "tesa_backward", "ssd_backward"};

} // namespace

void record_begin(hipStream_t s)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_error != hipSuccess) return;
    if (g_used == g_pairs.size()) {
        Pair p;
        hipError_t e = hipEventCreate(&p.begin);
        if (e == hipSuccess) e = hipEventCreate(&p.end);
        if (e != hipSuccess) {
            g_error = e;
            return;
        }
        g_pairs.push_back(p);
    }
    const hipError_t e = hipEventRecord(g_pairs[g_used].begin, s);
    if (e != hipSuccess) {
        g_error = e;
        return;
    }
    g_open = true;
}

void record_end(hipStream_t s)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_open) return;
    g_open = false;
    const hipError_t e = hipEventRecord(g_pairs[g_used].end, s);
    if (e != hipSuccess) {
        g_error = e;
        return;
    }
    ++g_used;
}

} // namespace timing
} // namespace mate

using namespace mate::timing;

extern "C" {

mate_status mate_timing_begin(const char *kernel)
{
    if (!kernel) return MATE_ERR_NULL;
    int id = -1;
    for (int i = 0; i < mate::K_COUNT; ++i)
        if (std::strcmp(kernel, kNames[i]) == 0) id = i;
    if (id < 0) return MATE_ERR_SHAPE;
    std::lock_guard<std::mutex> lk(g_mu);
    if (armed.load() >= 0) return MATE_ERR_SHAPE;
    g_used = 0;
    g_open = false;
    g_error = hipSuccess;
    armed.store(id);
    return MATE_OK;
}

mate_status mate_timing_end(int64_t *launches, double *total_ms)
{
    if (!launches || !total_ms) return MATE_ERR_NULL;
    armed.store(-1);
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_error != hipSuccess) return MATE_ERR_DEVICE;
    double sum = 0.0;
    for (size_t i = 0; i < g_used; ++i) {
        hipError_t e = hipEventSynchronize(g_pairs[i].end);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_pairs[i].begin, g_pairs[i].end);
        if (e != hipSuccess) return MATE_ERR_DEVICE;
        sum += ms;
    }
    *launches = (int64_t)g_used;
    *total_ms = sum;
    g_used = 0;
    return MATE_OK;
}

} // extern "C"
