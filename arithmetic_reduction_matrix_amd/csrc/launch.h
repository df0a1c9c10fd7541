// Kernel launchers (one per operation), called by the C entry points after
// the arguments have been checked and a Plan made.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "plan.h"

namespace armx {

// Workspace layout of the reductions with a completion ticket: a 256-byte
// counter region (top counter, then one per group of blocks), the block
// results, then the group results.
struct Workspace {
  unsigned* counters;
  float* partials;
  float* group_partials;
};

inline Workspace workspace_layout(const Plan& plan, void* ws) {
  char* base = static_cast<char*>(ws);
  Workspace w;
  w.counters = reinterpret_cast<unsigned*>(base);
  w.partials = reinterpret_cast<float*>(base + kCounterBytes);
  w.group_partials = reinterpret_cast<float*>(base + kCounterBytes + plan.partials_bytes);
  return w;
}

// Launches the main kernel of a plan.  When the plan carries events they are
// stamped by the kernel's own dispatch (start and completion) through
// hipExtLaunchKernel; otherwise it is a plain hipLaunchKernel, which stream
// capture (HIP graphs) records as an ordinary kernel node.
inline hipError_t launch_main(const Plan& plan, const void* fn, void** args, hipStream_t stream) {
  const dim3 grid(unsigned(plan.grid)), block(unsigned(plan.waves * 64));
  if (!plan.start_event && !plan.stop_event)
    return hipLaunchKernel(fn, grid, block, args, plan.lds_bytes, stream);
  return hipExtLaunchKernel(fn, grid, block, args, plan.lds_bytes, stream,
                            static_cast<hipEvent_t>(plan.start_event),
                            static_cast<hipEvent_t>(plan.stop_event), 0);
}

// out[0] = sum of x[0..plan.n); ws holds the counter and the block results.
hipError_t launch_sum(const Plan& plan, const void* x, float* out, void* ws, hipStream_t stream);

// out[0] = balanced-tree sum of x[0..plan.n).
hipError_t launch_fixed(const Plan& plan, const void* x, float* out, void* ws,
                        hipStream_t stream);

// out[r] = sum of row r, r < plan.rows.
hipError_t launch_rows(const Plan& plan, const void* x, float* out, hipStream_t stream);

// out[r] = balanced-tree sum of row r, r < plan.rows.
hipError_t launch_rows_fixed(const Plan& plan, const void* x, float* out, hipStream_t stream);

// out[0 .. count) = +0.0 (a small kernel rather than a memset, so the call can
// be captured in a graph and replayed).
hipError_t launch_zero(float* out, uint64_t count, hipStream_t stream);

}  // namespace armx
