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
//  * flat (many rows of at most 64 groups of R chunks, R a power of two):
//    each wavefront owns rows g, g + T, ...; it streams (row, group) items
//    with a software pipeline that runs across rows; a row's last group may
//    end inside the row, and its values past the row are -0.0 (read and
//    masked as load_row_chain and mask_row_chain describe; the last group of
//    the matrix's last row is read after the stream with load_last_chain,
//    which reads nothing past the row), so it is still the subtree
//    of its R-aligned chunks; a group's subtree root is selected
//    into lane (group index) of a slot register, and the row root is
//    lane_tree_full of that register (lanes past the row's groups hold -0.0,
//    which only passes values up), written after every group so that the
//    last write is the complete root.  The loop body branches only around
//    the masking of a row's last group.
//  * rows of at most 512 values go to the segmented kernel of
//    short_rows_kernels.hip.
//  * general (any length): each block sums a row; its W wavefronts (W a power
//    of two) take aligned power-of-two chunk ranges of the row and reduce
//    them as the flat fixed-order kernel does; the W roots are combined by a
//    lane tree.
//  * split (few rows, with a workspace): every row is cut into S aligned
//    ranges of 2^c chunks, one wavefront each in blocks spread over the
//    device; each range's subtree root is published, and the last block to
//    finish takes, for every row, the balanced tree over its S roots (padded
//    with -0.0), which is the row's tree above those subtrees.
// MMA selects the order with MFMA leaves (every chunk node one
// v_mfma_f32_16x16x32_f16 against ones and the tree over its 16 column sums,
// as for the flat fixed-order sum), per row.  A chunk that lies wholly past
// the row (the -0.0 reads of a partial last group) then has node +0.0 instead
// of -0.0: an MFMA from a zero accumulator never returns -0.0, so no node of
// the row's own chunks is -0.0, and adding +0.0 to such a node leaves it as it
// is, exactly as -0.0 would.
#include "fixed_tree.hpp"
#include "row_tail.hpp"
#include "launch.h"

namespace armx {
namespace {

using namespace dev;
using namespace dev::tree;

// Root of one loaded group (R chunks, R-aligned, R a power of two).
template <int R, bool MMA>
__device__ __forceinline__ float group_root(const u32x4 (&v)[R]) {
  if constexpr (MMA) {
    return group_node_mma<R>(v);
  } else if constexpr (R == 1) {
    return chunk_node(v[0]);
  } else {
    return group_node<R>(v);
  }
}

// PARTIAL: whether rows end inside a group (instantiated apart, so that whole
// groups carry no masking code at all).  RANGE (with PARTIAL, for rows of
// less than 2 GiB): the groups are read by load_row_chain_range, so nothing
// past a row's last 16-byte slot is fetched; the zeros it returns past the
// row are masked to -0.0 like the rest of the last group.
template <int R, bool NT, bool MMA, bool PARTIAL, bool RANGE = false>
__device__ __forceinline__ void rows_fixed_flat(const uint16_t* __restrict__ x, uint64_t rows,
                                                uint64_t cols, uint64_t ld,
                                                float* __restrict__ out, uint64_t g, uint64_t T,
                                                int lane) {
  if (g >= rows) return;
  const uint64_t group_elems = uint64_t(R) * 512;
  const uint64_t gpr = (cols + group_elems - 1) / group_elems;
  const uint64_t last_chunk = (cols - 1) / 512;
  const u32x4* fill = neg_zero_chunk();
  const uint32_t row_bytes = uint32_t((cols * 2 + 15) & ~uint64_t(15));
  u32x4 keep[R];
  if constexpr (PARTIAL) row_tail_keep<R>(cols, lane, keep);
  const uint64_t K = (rows - 1 - g) / T + 1;
  const bool last_apart = PARTIAL && g + (K - 1) * T == rows - 1;
  const uint64_t items = K * gpr - (last_apart ? 1 : 0);   // streamed (row, group) items
  const uint64_t row_step = T * ld;
  uint64_t lc = 0;           // group of the next item to load
  uint64_t rk = 0, rc = 0;   // next (row, group) to reduce
  uint64_t issued = 0;
  const uint16_t* load_row = x + g * ld;
  auto load = [&](u32x4 (&v)[R]) {
    if constexpr (RANGE) {
      load_row_chain_range<R, NT>(load_row, row_bytes, lc, lane, v);
    } else {
      load_row_chain_counted<R, NT, PARTIAL>(load_row, lc, last_chunk, fill, lane, v);
    }
    // stays on the last streamed item once it is reached (the re-read is not used)
    const bool more = ++issued < items;
    const bool more_in_row = lc + 1 < gpr;
    lc = more ? (more_in_row ? lc + 1 : 0) : lc;
    load_row = (more && !more_in_row) ? load_row + row_step : load_row;
  };
  float slots = -0.0f;
  auto reduce = [&](u32x4 (&v)[R]) {
    if constexpr (PARTIAL) {
      if (rc + 1 == gpr) apply_row_tail<R>(v, keep, 0x8000u);
    }
    const float node = group_root<R, MMA>(v);
    slots = uint64_t(lane) == rc ? node : (rc == 0 ? -0.0f : slots);
    const float root = lane_tree_full(slots);
    out[g + rk * T] = root;  // every group; the row's last group writes the root
    const bool row_done = rc + 1 == gpr;
    rc = row_done ? 0 : rc + 1;
    rk = row_done ? rk + 1 : rk;
  };
  // The last group of the matrix's last row: its loads go out first, with
  // the stream's first loads, and it is reduced after the stream.
  u32x4 fin[R];
  uint32_t fin_h[8];
  if constexpr (PARTIAL) {
    if (last_apart) load_last_chain<R, NT>(x + (rows - 1) * ld, gpr - 1, cols, lane, fin, fin_h);
  }
  if (items > 0) {
    u32x4 a[R], b[R];
    load(a);
    uint64_t j = 0;
    for (; j + 1 < items; j += 2) {
      load(b);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the reduction
      reduce(a);
      load(a);
      __builtin_amdgcn_sched_barrier(0);
      reduce(b);
    }
    if (j < items) reduce(a);
  }
  if constexpr (PARTIAL) {
    if (last_apart) {   // reduce() masks it and writes the row's root
      merge_last_chain<R>(fin, fin_h, gpr - 1, cols, lane);
      reduce(fin);
    }
  }
}

template <int R, bool NT, bool MMA>
__global__ __launch_bounds__(1024) void rows_fixed_kernel(const uint16_t* __restrict__ x,
                                                          uint64_t rows, uint64_t cols,
                                                          uint64_t ld, float* __restrict__ out,
                                                          int flat, int log2c,
                                                          unsigned slots_per_wave, int remap) {
  __shared__ float red[16];
  const int lane = lane_id();
  const int W = num_waves();

  if (flat) {
    if constexpr (is_pow2(R)) {
      const uint64_t g = (remap ? xcd_block_id() : uint64_t(blockIdx.x)) * W + wave_id();
      const uint64_t T = uint64_t(gridDim.x) * W;
      if (cols % (uint64_t(R) * 512) != 0) {
        rows_fixed_flat<R, NT, MMA, true, true>(x, rows, cols, ld, out, g, T, lane);
      } else {
        rows_fixed_flat<R, NT, MMA, false>(x, rows, cols, ld, out, g, T, lane);
      }
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
    const float wave_root =
        wave_range_root<R, NT, 0, MMA>(xr, cols, first, valid, lane, log_rows);
    __syncthreads();
    if (lane == 0) red[wave_id()] = wave_root;
    __syncthreads();
    if (wave_id() == 0) {
      const float root = lane_tree(lane < W ? red[lane] : -0.0f, lv);
      if (lane == 0) out[row] = root;
    }
  }
}

// Few rows: wavefront `item` (block * W + wave) reduces range s = item % S of
// row item / S (chunks s 2^log2c .. + 2^log2c, cut at the row's end, values
// past the row -0.0) to its subtree root, publishes it in partials[item],
// and the last block writes out[r] = the balanced tree over row r's S roots
// padded with -0.0 (combine_split_rows): the row's tree above its ranges.
template <int R, bool NT, bool MMA>
__global__ __launch_bounds__(1024) void rows_fixed_split_kernel(
    const uint16_t* __restrict__ x, uint64_t rows, uint64_t cols, uint64_t ld,
    float* __restrict__ out, unsigned segs, int log2c, unsigned slots_per_wave,
    unsigned* __restrict__ counter, float* __restrict__ partials) {
  __shared__ int flag;
  __shared__ float stage[kSplitMaxItems];
  extern __shared__ float node_lds[];
  const int lane = lane_id();
  const uint64_t W = uint64_t(num_waves());
  const uint64_t S = segs;
  const uint64_t item = uint64_t(blockIdx.x) * W + uint64_t(wave_id());
  if (item < rows * S) {
    const uint64_t row = item / S, s = item % S;
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * ld);
    const uint64_t chunks = (cols + 511) / 512;
    const uint64_t first = s << log2c;
    const uint64_t span = uint64_t(1) << log2c;
    const uint64_t valid = chunks - first < span ? chunks - first : span;
    float* log_rows = node_lds + unsigned(wave_id()) * slots_per_wave;
    const float root =
        valid / R >= kPaceLongChains
            ? wave_range_root<R, NT, 2, MMA>(xr, cols, first, valid, lane, log_rows)
            : wave_range_root<R, NT, 0, MMA>(xr, cols, first, valid, lane, log_rows);
    if (lane == 0) __hip_atomic_store(partials + item, root, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the root is stored
  }
  __syncthreads();   // every wavefront's root is stored before the block counts
  if (!publish_with_ticket([] {}, counter, gridDim.x, &flag)) return;
  combine_split_rows(partials, rows, segs, out, stage, unsigned(W) * 64);
}

template <int R>
const void* pick_rows_fixed(bool nt, bool mma) {
  if (mma)
    return nt ? reinterpret_cast<const void*>(&rows_fixed_kernel<R, true, true>)
              : reinterpret_cast<const void*>(&rows_fixed_kernel<R, false, true>);
  return nt ? reinterpret_cast<const void*>(&rows_fixed_kernel<R, true, false>)
            : reinterpret_cast<const void*>(&rows_fixed_kernel<R, false, false>);
}

const void* rows_fixed_kernel_for(int r, bool nt, bool mma) {
  switch (r) {
    case 1: return pick_rows_fixed<1>(nt, mma);
    case 2: return pick_rows_fixed<2>(nt, mma);
    case 3: return pick_rows_fixed<3>(nt, mma);
    case 4: return pick_rows_fixed<4>(nt, mma);
    case 5: return pick_rows_fixed<5>(nt, mma);
    case 6: return pick_rows_fixed<6>(nt, mma);
    case 7: return pick_rows_fixed<7>(nt, mma);
    case 8: return pick_rows_fixed<8>(nt, mma);
    default: return nullptr;
  }
}

template <int R>
const void* pick_split(bool nt, bool mma) {
  if (mma)
    return nt ? reinterpret_cast<const void*>(&rows_fixed_split_kernel<R, true, true>)
              : reinterpret_cast<const void*>(&rows_fixed_split_kernel<R, false, true>);
  return nt ? reinterpret_cast<const void*>(&rows_fixed_split_kernel<R, true, false>)
            : reinterpret_cast<const void*>(&rows_fixed_split_kernel<R, false, false>);
}

const void* rows_fixed_split_kernel_for(int r, bool nt, bool mma) {
  switch (r) {
    case 1: return pick_split<1>(nt, mma);
    case 2: return pick_split<2>(nt, mma);
    case 3: return pick_split<3>(nt, mma);
    case 4: return pick_split<4>(nt, mma);
    case 5: return pick_split<5>(nt, mma);
    case 6: return pick_split<6>(nt, mma);
    case 7: return pick_split<7>(nt, mma);
    case 8: return pick_split<8>(nt, mma);
    default: return nullptr;
  }
}

}  // namespace

hipError_t launch_rows_fixed(const Plan& plan, const void* x, float* out, void* ws,
                             hipStream_t stream) {
  if (plan.rows == 0) return hipSuccess;
  if (plan.n == 0) return launch_zero(out, plan.rows, stream);
  if (plan.mode == 2) return launch_short_rows(plan, x, out, stream);
  if (plan.mode == 3) {
    const void* fn = rows_fixed_split_kernel_for(plan.r,
                                                 (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0,
                                                 (plan.flags & ARMX_FLAG_MMA_LEAVES) != 0);
    if (!fn || !ws || plan.segs > kSplitMaxSegs || plan.rows * plan.segs > kSplitMaxItems)
      return hipErrorInvalidValue;   // more parts than the last block's stage and tree hold
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    uint64_t rows = plan.rows, cols = plan.n, ld = plan.ld;
    unsigned segs = plan.segs;
    int log2c = plan.log2_chunks;
    unsigned slots_per_wave = plan.slots_per_wave;
    Workspace w = workspace_layout(plan, ws);
    void* args[] = {&xh,  &rows,           &cols,       &ld,        &out,
                    &segs, &log2c, &slots_per_wave, &w.counters, &w.partials};
    return launch_main(plan, fn, args, stream);
  }
  const void* fn = rows_fixed_kernel_for(plan.r, (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0,
                                         (plan.flags & ARMX_FLAG_MMA_LEAVES) != 0);
  if (!fn) return hipErrorInvalidValue;
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  uint64_t rows = plan.rows, cols = plan.n, ld = plan.ld;
  int flat = plan.mode;
  int log2c = plan.log2_chunks;
  unsigned slots_per_wave = plan.slots_per_wave;
  int remap = plan.xcd_remap;
  void* args[] = {&xh, &rows, &cols, &ld, &out, &flat, &log2c, &slots_per_wave, &remap};
  return launch_main(plan, fn, args, stream);
}

}  // namespace armx
