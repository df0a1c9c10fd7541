// Fixed-order sum: one prescribed balanced binary tree, bitwise reproducible.
//
// "Taming Bitwise Behavior in GPU Kernels with Tensor Core" (arXiv
// 2609.11356), Abstract: the order of a floating-point reduction is the main
// reason two deterministic kernels disagree bit for bit, next to partial-sum
// precision, fused multiply-add and rounding placement; enforcing a
// balanced-tree order makes the result independent of tile shapes.
// "GPU Tensor Cores for fast Arithmetic Reductions" (arXiv 2001.05585),
// Abstract: partial results are 32-bit floats.
//
// The tree: leaves x[i] widened exactly to binary32, padded with -0.0 to a
// power of two (x + -0.0 == x for every x, so padding only passes values up);
// each node is one binary32 round-to-nearest-even addition of its children.
// Only v_add_f32 is used -- no MFMA, whose internal accumulation order and
// rounding are not specified, and no fused multiply-add.
//
// How the GPU walks it:
//  * chunk = one wavefront load, 512 values = two 256-value leaf tiles, an
//    aligned depth-9 subtree.  Lane l holds leaves [8l, 8l + 8): in-lane
//    levels 1-3, then lane_tree levels 4-9 (lane ^ 1, ^ 2, ^ 4, ^ 8, ^ 16,
//    ^ 32).  Every lane ends with the chunk's node value.
//  * wavefront = an aligned range of 2^c chunks.  Chunk nodes are merged in
//    index order with a binary counter: after chunk k, stack level j holds
//    the node of the last complete group of 2^j chunks.  Chunks past the end
//    of the input are never loaded; they would be -0.0 subtrees.
//  * block = W (a power of two) consecutive wavefront ranges, combined by a
//    lane_tree over W lanes; the block result is an aligned subtree.
//  * grid: the block results are combined by the same tree (padded with
//    -0.0): groups of a power-of-two number of consecutive blocks are
//    complete subtrees, combined by the last block of each group, and the
//    group results by the last group (or all of it by a second launch).
// The chain length R only sets how many chunk loads a wavefront has in
// flight; it never changes which values are added together.
#include "fixed_tree.hpp"
#include "launch.h"

namespace armx {
namespace {

using namespace dev;
using namespace dev::tree;

template <int R, bool NT, bool MMA>
__global__ __launch_bounds__(1024) void fixed_kernel(const u32x4* __restrict__ x, uint64_t n,
                                                     int log2c, unsigned slots_per_wave,
                                                     unsigned* __restrict__ counters,
                                                     float* __restrict__ roots,
                                                     float* __restrict__ group_roots,
                                                     unsigned group, float* __restrict__ out,
                                                     int two_pass) {
  __shared__ float red[16];
  __shared__ int flag;
  const int lane = lane_id();
  const int W = num_waves();
  const uint64_t chunks = (n + 511) / 512;
  const uint64_t first = (uint64_t(blockIdx.x) * W + uint64_t(wave_id())) << log2c;
  const uint64_t span = uint64_t(1) << log2c;
  const uint64_t valid = first >= chunks ? 0 : (chunks - first < span ? chunks - first : span);

  // This wavefront's node log in dynamic LDS (`slots_per_wave` floats each).
  // Long ranges pace their stream (pace_pause; measured on MI355X: PACE 2 from
  // 64 groups of R chunks per wavefront).
  extern __shared__ float node_lds[];
  float* log_rows = node_lds + unsigned(wave_id()) * slots_per_wave;
  const float wave_root =
      valid / R >= kPaceLongChains
          ? wave_range_root<R, NT, 2, MMA>(x, n, first, valid, lane, log_rows)
          : wave_range_root<R, NT, 0, MMA>(x, n, first, valid, lane, log_rows);

  // block: W consecutive wavefront subtrees -> one subtree
  __syncthreads();
  if (lane == 0) red[wave_id()] = wave_root;
  __syncthreads();
  float block_root = -0.0f;
  if (wave_id() == 0) {
    float v = lane < W ? red[lane] : -0.0f;
    int lv = 0;
    while ((1 << lv) < W) ++lv;
    block_root = lane_tree(v, lv);
  }

  if (gridDim.x == 1) {
    if (threadIdx.x == 0) out[0] = block_root;
    return;
  }
  if (two_pass) {
    if (threadIdx.x == 0) roots[blockIdx.x] = block_root;
    return;
  }
  // groups are aligned power-of-two runs of blocks: complete subtrees
  const unsigned T = unsigned(W) * 64;
  finish_two_level(block_root, counters, roots, group_roots, group, out, red, &flag,
                   [T](const float* v, unsigned c, float* r) { return tree_of_values(v, c, r, T); },
                   span < kSplitCountChains * R);
}

__global__ __launch_bounds__(1024) void fixed_final_kernel(const float* __restrict__ roots,
                                                           unsigned count,
                                                           float* __restrict__ out) {
  __shared__ float red[16];
  const float root = tree_of_values(roots, count, red, blockDim.x);
  if (threadIdx.x == 0) out[0] = root;
}

template <int R>
const void* pick_fixed(bool nt, bool mma) {
  if (mma)
    return nt ? reinterpret_cast<const void*>(&fixed_kernel<R, true, true>)
              : reinterpret_cast<const void*>(&fixed_kernel<R, false, true>);
  return nt ? reinterpret_cast<const void*>(&fixed_kernel<R, true, false>)
            : reinterpret_cast<const void*>(&fixed_kernel<R, false, false>);
}

const void* fixed_kernel_for(int r, bool nt, bool mma) {
  switch (r) {
    case 1: return pick_fixed<1>(nt, mma);
    case 2: return pick_fixed<2>(nt, mma);
    case 3: return pick_fixed<3>(nt, mma);
    case 4: return pick_fixed<4>(nt, mma);
    case 5: return pick_fixed<5>(nt, mma);
    case 6: return pick_fixed<6>(nt, mma);
    case 7: return pick_fixed<7>(nt, mma);
    case 8: return pick_fixed<8>(nt, mma);
    default: return nullptr;
  }
}

}  // namespace

hipError_t launch_fixed(const Plan& plan, const void* x, float* out, void* ws,
                        hipStream_t stream) {
  if (plan.n == 0) return launch_zero(out, 1, stream);
  const void* fn = fixed_kernel_for(plan.r, (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0,
                                    (plan.flags & ARMX_FLAG_MMA_LEAVES) != 0);
  if (!fn) return hipErrorInvalidValue;
  const u32x4* xv = static_cast<const u32x4*>(x);
  uint64_t n = plan.n;
  int log2c = plan.log2_chunks;
  unsigned slots_per_wave = plan.slots_per_wave;
  Workspace w = workspace_layout(plan, ws);
  unsigned group = plan.group;
  int two_pass = (plan.flags & ARMX_FLAG_TWO_PASS) ? 1 : 0;
  void* args[] = {&xv, &n, &log2c, &slots_per_wave, &w.counters, &w.partials, &w.group_partials,
                  &group, &out, &two_pass};
  hipError_t e = launch_main(plan, fn, args, stream);
  if (e != hipSuccess || !two_pass || plan.grid == 1) return e;
  unsigned count = unsigned(plan.grid);
  const float* croots = w.partials;
  // the final tree needs a power-of-two block: 1024 threads
  void* fargs[] = {&croots, &count, &out};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fixed_final_kernel), dim3(1), dim3(1024),
                         fargs, 0, stream);
}

}  // namespace armx
