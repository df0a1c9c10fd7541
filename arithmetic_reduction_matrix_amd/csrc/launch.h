// Kernel launchers (one per operation), called by the C entry points after
// the arguments have been checked and a Plan made.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace armx {

// out[0] = sum of x[0..plan.n); ws holds the counter and the block results.
hipError_t launch_sum(const Plan& plan, const void* x, float* out, void* ws, hipStream_t stream);

// out[0] = balanced-tree sum of x[0..plan.n).
hipError_t launch_fixed(const Plan& plan, const void* x, float* out, void* ws,
                        hipStream_t stream);

// out[r] = sum of row r, r < plan.rows.
hipError_t launch_rows(const Plan& plan, const void* x, float* out, hipStream_t stream);

// out[0 .. count) = +0.0 (a small kernel rather than a memset, so the call can
// be captured in a graph and replayed).
hipError_t launch_zero(float* out, uint64_t count, hipStream_t stream);

}  // namespace armx
