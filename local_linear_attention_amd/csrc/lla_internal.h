// Internal declarations shared by the liblla translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lla {

struct Problem {
    const void* q;
    const void* k;
    const void* v;
    float* out;
    int64_t B, H, n, d;
    double h, lambda;
    int dtype;            // 0 = f32, 1 = bf16
    hipStream_t stream;
};

// fp64-accumulating path: every (dtype, d) the library accepts.
hipError_t launch_exact(const Problem& p);

// Matrix-core path for bf16 inputs.  Returns hipErrorNotSupported when (dtype, d) is not
// covered, before launching anything.
bool fast_supports(int dtype, int64_t d);
hipError_t launch_fast(const Problem& p);

}  // namespace lla
