// Per-kernel HIP event timing (the mate_timing_* diagnostics).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace mate {

enum KernelId : int {
    K_RMS_REORDER = 0,
    K_SSD_POOL,
    K_SSD_PREP,
    K_SSD_CB,
    K_SSD_STATES,
    K_SSD_SEG_PASS,
    K_SSD_OUT,
    K_TESA,
    K_MAMBA,
    K_TESA_BWD,
    K_SSD_BWD,
    K_COUNT
};

namespace timing {

extern std::atomic<int> armed;  // kernel id being timed, -1 when none

void record_begin(hipStream_t s);
void record_end(hipStream_t s);

// Brackets one launch of kernel `id` with an event pair when that kernel is armed.
struct Scope {
    hipStream_t stream;
    bool on;
    Scope(KernelId id, hipStream_t s) : stream(s), on(armed.load(std::memory_order_relaxed) == (int)id)
    {
        if (on) record_begin(stream);
    }
    ~Scope()
    {
        if (on) record_end(stream);
    }
};

} // namespace timing
} // namespace mate
