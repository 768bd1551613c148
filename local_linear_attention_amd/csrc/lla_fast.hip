// Matrix-core path for bf16 inputs (not yet available: every request falls back to the
// fp64 path under LLA_PATH_AUTO and is refused under LLA_PATH_FAST).
#include "lla_internal.h"

namespace lla {

bool fast_supports(int, int64_t) { return false; }

hipError_t launch_fast(const Problem&) { return hipErrorNotSupported; }

}  // namespace lla
