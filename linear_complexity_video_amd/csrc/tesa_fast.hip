// MFMA path of TESA (not built yet: every shape uses the portable kernel).
#include "launch.hpp"

namespace mate {
bool tesa_fast_supports(const TesaProblem &) { return false; }
hipError_t tesa_fast(const TesaProblem &, const TesaArgs &, hipStream_t) { return hipErrorNotSupported; }
} // namespace mate
