// MFMA path of the bidirectional scan (not built yet: every shape uses the portable kernels).
#include "launch.hpp"

namespace mate {
bool ssd_fast_supports(const SsdProblem &) { return false; }
size_t ssd_fast_workspace(const SsdProblem &) { return 0; }
hipError_t ssd_fast(const SsdProblem &, const SsdArgs &, void *, hipStream_t) { return hipErrorNotSupported; }
hipError_t ssd_fast_prepare() { return hipSuccess; }
} // namespace mate
