// Row-segmented fixed-order sums: out[r] = the balanced-tree sum of row r.
//
// Each row's result is the root of the balanced binary tree over that row's
// cols values (padded with -0.0 to a power of two, every node one binary32
// round-to-nearest-even addition) -- the order that "Taming Bitwise Behavior
// in GPU Kernels with Tensor Core" (arXiv 2609.11356, Abstract) enforces to
// make reductions reproducible, applied per row.  It depends on the row's
// values only: not on how many rows there are, where the row sits, the block
// size, the chain length or the grid -- the batch invariance that tile-shape
// choices otherwise break (same Abstract).
//
// Two mappings:
//  * flat (many rows whose length is a whole number of R-chunk groups, at
//    most 64 groups): each wavefront owns rows g, g + T, ...; it streams
//    (row, group) items with a software pipeline that runs across rows; a
//    group's subtree root is selected into lane (group index) of a slot
//    register, and the row root is lane_tree_full of that register (lanes
//    past the row's groups hold -0.0, which only passes values up), written
//    after every group so that the last write is the complete root.  The
//    loop body has no branches.
//  * general (any length): each block sums a row; its W wavefronts (W a power
//    of two) take aligned power-of-two chunk ranges of the row and reduce
//    them as the flat fixed-order kernel does; the W roots are combined by a
//    lane tree.
#include "fixed_tree.hpp"
#include "launch.h"

namespace armx {
namespace {

using namespace dev;
using namespace dev::tree;

// Root of one loaded group (R chunks, R-aligned, R a power of two).
template <int R>
__device__ __forceinline__ float group_root(const u32x4 (&v)[R]) {
  if constexpr (R == 1) {
    return chunk_node(v[0]);
  } else {
    return group_node<R>(v);
  }
}

template <int R, bool NT>
__device__ __forceinline__ void rows_fixed_flat(const uint16_t* __restrict__ x, uint64_t rows,
                                                uint64_t gpr, uint64_t ld,
                                                float* __restrict__ out, uint64_t g, uint64_t T,
                                                int lane) {
  if (g >= rows) return;
  const uint64_t K = (rows - 1 - g) / T + 1;
  const uint64_t items = K * gpr;
  uint64_t lk = 0, lc = 0;   // next (row, group) to load
  uint64_t rk = 0, rc = 0;   // next (row, group) to reduce
  auto ptr = [&]() {
    return reinterpret_cast<const u32x4*>(x + (g + lk * T) * ld) + lc * (uint64_t(R) * 64);
  };
  auto advance_load = [&]() {
    // stays on the last item once it is reached (the re-read is not used)
    const bool more_in_row = lc + 1 < gpr;
    const bool more_rows = lk + 1 < K;
    lc = more_in_row ? lc + 1 : (more_rows ? 0 : lc);
    lk = more_in_row ? lk : (more_rows ? lk + 1 : lk);
  };
  float slots = -0.0f;
  auto reduce = [&](const u32x4 (&v)[R]) {
    const float node = group_root<R>(v);
    slots = uint64_t(lane) == rc ? node : (rc == 0 ? -0.0f : slots);
    const float root = lane_tree_full(slots);
    out[g + rk * T] = root;  // every group; the row's last group writes the root
    const bool row_done = rc + 1 == gpr;
    rc = row_done ? 0 : rc + 1;
    rk = row_done ? rk + 1 : rk;
  };
  u32x4 a[R], b[R];
  load_group<R, NT>(ptr(), 0, lane, a);
  advance_load();
  uint64_t j = 0;
  for (; j + 1 < items; j += 2) {
    load_group<R, NT>(ptr(), 0, lane, b);
    advance_load();
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the reduction
    reduce(a);
    load_group<R, NT>(ptr(), 0, lane, a);
    advance_load();
    __builtin_amdgcn_sched_barrier(0);
    reduce(b);
  }
  if (j < items) reduce(a);
}

template <int R, bool NT>
__global__ __launch_bounds__(1024) void rows_fixed_kernel(const uint16_t* __restrict__ x,
                                                          uint64_t rows, uint64_t cols,
                                                          uint64_t ld, float* __restrict__ out,
                                                          int flat, int log2c,
                                                          unsigned slots_per_wave) {
  __shared__ float red[16];
  const int lane = lane_id();
  const int W = num_waves();

  if (flat) {
    if constexpr (is_pow2(R)) {
      const uint64_t gpr = cols / (uint64_t(R) * 512);
      rows_fixed_flat<R, NT>(x, rows, gpr, ld, out, uint64_t(blockIdx.x) * W + wave_id(),
                             uint64_t(gridDim.x) * W, lane);
    }
    return;
  }

  extern __shared__ float node_lds[];
  float* log_rows = node_lds + unsigned(wave_id()) * slots_per_wave;
  const uint64_t chunks = (cols + 511) / 512;
  const uint64_t first = uint64_t(wave_id()) << log2c;
  const uint64_t span = uint64_t(1) << log2c;
  const uint64_t valid = first >= chunks ? 0 : (chunks - first < span ? chunks - first : span);
  int lv = 0;
  while ((1 << lv) < W) ++lv;
  for (uint64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * ld);
    const float wave_root = wave_range_root<R, NT>(xr, cols, first, valid, lane, log_rows);
    __syncthreads();
    if (lane == 0) red[wave_id()] = wave_root;
    __syncthreads();
    if (wave_id() == 0) {
      const float root = lane_tree(lane < W ? red[lane] : -0.0f, lv);
      if (lane == 0) out[row] = root;
    }
  }
}

template <int R>
const void* pick_rows_fixed(bool nt) {
  return nt ? reinterpret_cast<const void*>(&rows_fixed_kernel<R, true>)
            : reinterpret_cast<const void*>(&rows_fixed_kernel<R, false>);
}

const void* rows_fixed_kernel_for(int r, bool nt) {
  switch (r) {
    case 1: return pick_rows_fixed<1>(nt);
    case 2: return pick_rows_fixed<2>(nt);
    case 3: return pick_rows_fixed<3>(nt);
    case 4: return pick_rows_fixed<4>(nt);
    case 5: return pick_rows_fixed<5>(nt);
    case 6: return pick_rows_fixed<6>(nt);
    case 7: return pick_rows_fixed<7>(nt);
    case 8: return pick_rows_fixed<8>(nt);
    default: return nullptr;
  }
}

}  // namespace

hipError_t launch_rows_fixed(const Plan& plan, const void* x, float* out, hipStream_t stream) {
  if (plan.rows == 0) return hipSuccess;
  if (plan.n == 0) return launch_zero(out, plan.rows, stream);
  const void* fn = rows_fixed_kernel_for(plan.r, (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0);
  if (!fn) return hipErrorInvalidValue;
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  uint64_t rows = plan.rows, cols = plan.n, ld = plan.ld;
  int flat = plan.mode;
  int log2c = plan.log2_chunks;
  unsigned slots_per_wave = plan.slots_per_wave;
  void* args[] = {&xh, &rows, &cols, &ld, &out, &flat, &log2c, &slots_per_wave};
  return launch_main(plan, fn, args, stream);
}

}  // namespace armx
