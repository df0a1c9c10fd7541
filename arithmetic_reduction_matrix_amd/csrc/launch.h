// Kernel launchers (one per operation), called by the C entry points after
// the arguments have been checked and a Plan made.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "plan.h"

namespace armx {

// Workspace layout of the reductions with a completion ticket: the counter
// region (kCounterBytes: the top counter, then one per group of blocks, each
// in its own 256-byte stretch), the block results, then the group results.
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

// Launches a kernel.  Events, when given, are stamped by the kernel's own
// dispatch (start and completion) through hipExtLaunchKernel; without them it
// is a plain hipLaunchKernel, which stream capture (HIP graphs) records as an
// ordinary kernel node.
inline hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, size_t lds,
                                hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (!start && !stop) return hipLaunchKernel(fn, grid, block, args, lds, stream);
  return hipExtLaunchKernel(fn, grid, block, args, lds, stream, start, stop, 0);
}

// Launches the main kernel of a plan, stamping the plan's events if any.
inline hipError_t launch_main(const Plan& plan, const void* fn, void** args, hipStream_t stream) {
  return launch_kernel(fn, dim3(unsigned(plan.grid)), dim3(unsigned(plan.waves * 64)), args,
                       plan.lds_bytes, stream, static_cast<hipEvent_t>(plan.start_event),
                       static_cast<hipEvent_t>(plan.stop_event));
}

// out[0] = sum of x[0..plan.n); ws holds the counter and the block results.
hipError_t launch_sum(const Plan& plan, const void* x, float* out, void* ws, hipStream_t stream);

// out[0] = sum of x[0..plan.n) by levels of MMA-only chain reductions, one
// launch per level; ws holds the level buffers after its counter region.
// The plan's start event is stamped by the first launch, its stop event by
// the last.
hipError_t launch_levels(const Plan& plan, const void* x, float* out, void* ws,
                         hipStream_t stream);

// out[0] = the binary32 nearest to the exact sum of x[0..plan.n); out_fixed
// (may be null) = that sum as a 128-bit count of 2^-24 (low word, high word).
hipError_t launch_exact(const Plan& plan, const void* x, float* out, int64_t* out_fixed,
                        void* ws, hipStream_t stream);

// out[0] = balanced-tree sum of x[0..plan.n).
hipError_t launch_fixed(const Plan& plan, const void* x, float* out, void* ws,
                        hipStream_t stream);

// out[r] = sum of row r, r < plan.rows; ws (the counter and the segment
// partials) is used by plan mode 3 only.
hipError_t launch_rows(const Plan& plan, const void* x, float* out, void* ws,
                       hipStream_t stream);

// out[r] = balanced-tree sum of row r, r < plan.rows; ws as for launch_rows.
hipError_t launch_rows_fixed(const Plan& plan, const void* x, float* out, void* ws,
                             hipStream_t stream);

// out[r] = balanced-tree sum of row r, r < plan.rows, for rows of at most one
// chunk (plan mode 2); serves both row entry points.
hipError_t launch_short_rows(const Plan& plan, const void* x, float* out, hipStream_t stream);

// out[0 .. count) = +0.0 (a small kernel rather than a memset, so the call can
// be captured in a graph and replayed).
hipError_t launch_zero(float* out, uint64_t count, hipStream_t stream);

// Device address, on the current device, of the static scratch array that
// reduce_sum_noalloc uses as its workspace (kScratchBytes bytes, 256-byte
// aligned); looked up with hipGetSymbolAddress on the first call per device.
hipError_t scratch_address(void** ptr);

}  // namespace armx
