// The C entry points declared in include/armx.h: check arguments, make a
// plan, enqueue kernels on the caller's stream.  Nothing here allocates.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "armx.h"
#include "launch.h"
#include "plan.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (cached); 256 if no device is usable.
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int cached = g_cu_count[dev].load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_ws(const armx::Plan& plan, const void* ws, size_t ws_bytes) {
  if (plan.ws_bytes == 0) return ARMX_OK;
  if (!ws) return ARMX_ERR_NULL;
  if (!aligned(ws, 256)) return ARMX_ERR_ALIGN;
  if (ws_bytes < plan.ws_bytes) return ARMX_ERR_WORKSPACE;
  return ARMX_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ARMX_OK : ARMX_ERR_HIP; }

// With the environment variable ARMX_LOG set (to anything), every accepted
// call writes its launch plan to stderr; otherwise the library never prints.
bool log_enabled() {
  static const bool on = std::getenv("ARMX_LOG") != nullptr;
  return on;
}

void log_plan(const char* entry, const armx::Plan& p) {
  if (!log_enabled()) return;
  std::fprintf(stderr,
               "armx: %s n=%llu rows=%llu ld=%llu grid=%d block=%d R=%d flags=0x%x "
               "mode=%d lds=%zu ws=%zu group=%u seg=%d remap=%d\n",
               entry, (unsigned long long)p.n, (unsigned long long)p.rows,
               (unsigned long long)p.ld, p.grid, p.waves * 64, p.r, p.flags, p.mode, p.lds_bytes,
               p.ws_bytes, p.group, p.seg_log2, p.xcd_remap);
}

// Common checks of reduce_sum, reduce_sum_fixed_order and reduce_sum_exact.
int prepare_flat(int op, const void* x, size_t n, float* out, void* ws, size_t ws_bytes,
                 const armx_config* cfg, armx::Plan* plan) {
  if (!out) return ARMX_ERR_NULL;
  if (n > 0 && !x) return ARMX_ERR_NULL;
  if (n > 0 && !aligned(x, 16)) return ARMX_ERR_ALIGN;
  // configuration errors are reported before touching the device
  armx::Plan probe;
  int st = armx::make_plan(op, n, 0, 0, cfg, 256, &probe);
  if (st != ARMX_OK) return st;
  st = armx::make_plan(op, n, 0, 0, cfg, n > 0 ? current_cu_count() : 256, plan);
  if (st != ARMX_OK) return st;
  return check_ws(*plan, ws, ws_bytes);
}

// Common checks and planning of the two row entry points.  The plans may
// split few long rows, or the last round of a row stream, over wavefronts of
// several blocks, which needs the workspace; without one (ws NULL) they are
// made without splits.
int prepare_rows(int op, const void* x, size_t rows, size_t cols, size_t ld, float* out,
                 void* ws, size_t ws_bytes, const armx_config* cfg, armx::RowPlans* plans) {
  if (rows > 0 && !out) return ARMX_ERR_NULL;
  if (rows > 0 && cols > 0 && !x) return ARMX_ERR_NULL;
  if (rows > 0 && cols > 0 && !aligned(x, 16)) return ARMX_ERR_ALIGN;
  // configuration errors are reported before touching the device
  armx::Plan probe;
  int st = armx::make_plan(op, rows, cols, ld, cfg, 256, &probe);
  if (st != ARMX_OK) return st;
  const int cus = rows > 0 && cols > 0 ? current_cu_count() : 256;
  st = armx::make_row_plans(op, rows, cols, ld, cfg, cus, plans, ws != nullptr);
  if (st != ARMX_OK) return st;
  armx::Plan need = plans->tail_rows ? plans->tail : plans->main;
  need.ws_bytes = plans->ws_bytes();
  return check_ws(need, ws, ws_bytes);
}

// Launches a row call's plans: the main one on the first rows, the tail (if
// any) on the last tail_rows rows.
template <class Launch>
hipError_t launch_row_plans(const armx::RowPlans& plans, const void* x, float* out, void* ws,
                            hipStream_t stream, Launch launch) {
  const uint64_t head = plans.main.rows;
  hipError_t e = launch(plans.main, x, out, ws, stream);
  if (e != hipSuccess || plans.tail_rows == 0) return e;
  const uint16_t* tx = static_cast<const uint16_t*>(x) + head * plans.main.ld;
  return launch(plans.tail, tx, out + head, ws, stream);
}

void log_row_plans(const char* entry, const armx::RowPlans& plans) {
  log_plan(entry, plans.main);
  if (plans.tail_rows) log_plan(entry, plans.tail);
}

}  // namespace

extern "C" {

int reduce_sum(const void* x, size_t n, float* out, void* ws, size_t ws_bytes,
               const armx_config* cfg, void* stream) {
  armx::Plan plan;
  int st = prepare_flat(armx::kOpSum, x, n, out, ws, ws_bytes, cfg, &plan);
  if (st != ARMX_OK) return st;
  log_plan("reduce_sum", plan);
  if (plan.flags & ARMX_FLAG_MMA_LEVELS)
    return hip_status(armx::launch_levels(plan, x, out, ws, static_cast<hipStream_t>(stream)));
  return hip_status(armx::launch_sum(plan, x, out, ws, static_cast<hipStream_t>(stream)));
}

int reduce_sum_noalloc(const void* x, size_t n, float* out, const armx_config* cfg,
                       void* stream) {
  armx::Plan plan;
  if (!out) return ARMX_ERR_NULL;
  if (n > 0 && !x) return ARMX_ERR_NULL;
  if (n > 0 && !aligned(x, 16)) return ARMX_ERR_ALIGN;
  int st = armx::make_plan(armx::kOpSum, n, 0, 0, cfg, 256, &plan);
  if (st != ARMX_OK) return st;
  st = armx::make_plan(armx::kOpSum, n, 0, 0, cfg, n > 0 ? current_cu_count() : 256, &plan);
  if (st != ARMX_OK) return st;
  if (plan.ws_bytes > armx::kScratchBytes) return ARMX_ERR_WORKSPACE;
  log_plan("reduce_sum_noalloc", plan);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    if (armx::scratch_address(&ws) != hipSuccess) return ARMX_ERR_HIP;
    // the completion counters the plan uses (the top counter and one per
    // group, each kCounterStride words apart; with one group, one per run of
    // kSplitCountRun blocks when the kernel splits its counting) must start
    // at zero: cleared by a small kernel on the caller's stream (capturable;
    // no memset, no allocation)
    uint64_t groups = plan.group ? (uint64_t(plan.grid) + plan.group - 1) / plan.group : 0;
    if (groups == 1)
      groups = (uint64_t(plan.grid) + armx::kSplitCountRun - 1) / armx::kSplitCountRun;
    const uint64_t words = (1 + groups) * armx::kCounterStride;
    const hipError_t e = armx::launch_zero(
        static_cast<float*>(ws),
        size_t(words < armx::kCounterBytes / 4 ? words : armx::kCounterBytes / 4), s);
    if (e != hipSuccess) return ARMX_ERR_HIP;
  }
  if (plan.flags & ARMX_FLAG_MMA_LEVELS)
    return hip_status(armx::launch_levels(plan, x, out, ws, s));
  return hip_status(armx::launch_sum(plan, x, out, ws, s));
}

int reduce_sum_fixed_order(const void* x, size_t n, float* out, void* ws, size_t ws_bytes,
                           const armx_config* cfg, void* stream) {
  armx::Plan plan;
  int st = prepare_flat(armx::kOpFixed, x, n, out, ws, ws_bytes, cfg, &plan);
  if (st != ARMX_OK) return st;
  log_plan("reduce_sum_fixed_order", plan);
  return hip_status(armx::launch_fixed(plan, x, out, ws, static_cast<hipStream_t>(stream)));
}

int reduce_sum_exact(const void* x, size_t n, float* out, int64_t* out_fixed, void* ws,
                     size_t ws_bytes, const armx_config* cfg, void* stream) {
  armx::Plan plan;
  int st = prepare_flat(armx::kOpExact, x, n, out, ws, ws_bytes, cfg, &plan);
  if (st != ARMX_OK) return st;
  if (out_fixed && !aligned(out_fixed, 8)) return ARMX_ERR_ALIGN;
  log_plan("reduce_sum_exact", plan);
  return hip_status(
      armx::launch_exact(plan, x, out, out_fixed, ws, static_cast<hipStream_t>(stream)));
}

int reduce_rows(const void* x, size_t rows, size_t cols, size_t ld, float* out, void* ws,
                size_t ws_bytes, const armx_config* cfg, void* stream) {
  armx::RowPlans plans;
  const int st = prepare_rows(armx::kOpRows, x, rows, cols, ld, out, ws, ws_bytes, cfg, &plans);
  if (st != ARMX_OK) return st;
  log_row_plans("reduce_rows", plans);
  return hip_status(launch_row_plans(plans, x, out, ws, static_cast<hipStream_t>(stream),
                                     armx::launch_rows));
}

int reduce_rows_fixed_order(const void* x, size_t rows, size_t cols, size_t ld, float* out,
                            void* ws, size_t ws_bytes, const armx_config* cfg, void* stream) {
  armx::RowPlans plans;
  const int st =
      prepare_rows(armx::kOpRowsFixed, x, rows, cols, ld, out, ws, ws_bytes, cfg, &plans);
  if (st != ARMX_OK) return st;
  log_row_plans("reduce_rows_fixed_order", plans);
  return hip_status(launch_row_plans(plans, x, out, ws, static_cast<hipStream_t>(stream),
                                     armx::launch_rows_fixed));
}

size_t armx_workspace_bytes(int op, size_t n_or_rows, size_t cols, const armx_config* cfg) {
  armx::Plan plan;
  if (op != ARMX_OP_SUM && op != ARMX_OP_ROWS && op != ARMX_OP_FIXED &&
      op != ARMX_OP_ROWS_FIXED && op != ARMX_OP_EXACT)
    return size_t(-1);
  const bool rows_op = op == ARMX_OP_ROWS || op == ARMX_OP_ROWS_FIXED;
  const bool empty = n_or_rows == 0 || (rows_op && cols == 0);
  const int cus = empty ? 256 : current_cu_count();
  // the row pitch does not change the workspace; take the smallest valid one
  const size_t ld = rows_op && n_or_rows > 1 ? (cols + 7) / 8 * 8 : cols;
  if (rows_op) {
    armx::RowPlans plans;
    if (armx::make_row_plans(op, n_or_rows, cols, ld, cfg, cus, &plans) != ARMX_OK)
      return size_t(-1);
    return plans.ws_bytes();
  }
  if (armx::make_plan(op, n_or_rows, cols, ld, cfg, cus, &plan) != ARMX_OK) return size_t(-1);
  return plan.ws_bytes;
}

int armx_launch_plan(int op, size_t n_or_rows, size_t cols, const armx_config* cfg,
                     armx_plan_info* info) {
  if (!info) return ARMX_ERR_NULL;
  if (op != ARMX_OP_SUM && op != ARMX_OP_ROWS && op != ARMX_OP_FIXED &&
      op != ARMX_OP_ROWS_FIXED && op != ARMX_OP_EXACT)
    return ARMX_ERR_CONFIG;
  const bool rows_op = op == ARMX_OP_ROWS || op == ARMX_OP_ROWS_FIXED;
  const bool empty = n_or_rows == 0 || (rows_op && cols == 0);
  const int cus = empty ? 256 : current_cu_count();
  const size_t ld = rows_op && n_or_rows > 1 ? (cols + 7) / 8 * 8 : cols;
  armx::RowPlans plans;
  int st;
  if (rows_op) {
    st = armx::make_row_plans(op, n_or_rows, cols, ld, cfg, cus, &plans);
  } else {
    st = armx::make_plan(op, n_or_rows, cols, ld, cfg, cus, &plans.main);
  }
  if (st != ARMX_OK) return st;
  const armx::Plan& p = plans.main;
  armx_plan_info r{};
  r.workspace_bytes = plans.ws_bytes();
  if (rows_op && n_or_rows == 0) {
    r.launches = 0;   // nothing to write
  } else if (empty) {
    r.launches = 1;   // the zero-fill kernel
  } else {
    r.grid_blocks = p.grid;
    r.block_threads = p.waves * 64;
    r.chain_r = p.r;
    r.lds_bytes = p.lds_bytes;
    r.waves_per_cu = double(p.grid) * double(p.waves) / double(cus);
    r.launches = 1;
    if (rows_op) {
      r.launches += plans.tail_rows ? 1 : 0;
    } else if (p.flags & ARMX_FLAG_MMA_LEVELS) {
      for (uint64_t c = armx::level_count(p.n, uint64_t(p.r), 1); c > 1;
           c = armx::level_count(c, uint64_t(p.r), 2))
        ++r.launches;
    } else if ((p.flags & ARMX_FLAG_TWO_PASS) && p.grid > 1) {
      ++r.launches;
    }
  }
  *info = r;
  return ARMX_OK;
}

const char* armx_status_string(int status) {
  switch (status) {
    case ARMX_OK: return "ARMX_OK";
    case ARMX_ERR_NULL: return "ARMX_ERR_NULL: a required pointer is NULL";
    case ARMX_ERR_ALIGN: return "ARMX_ERR_ALIGN: misaligned pointer or row pitch";
    case ARMX_ERR_CONFIG: return "ARMX_ERR_CONFIG: invalid block size, chain length, grid or flags";
    case ARMX_ERR_WORKSPACE: return "ARMX_ERR_WORKSPACE: workspace too small";
    case ARMX_ERR_SHAPE: return "ARMX_ERR_SHAPE: invalid or too large sizes";
    case ARMX_ERR_HIP: return "ARMX_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown armx status";
  }
}

int armx_version(void) { return 8; }

}  // extern "C"
