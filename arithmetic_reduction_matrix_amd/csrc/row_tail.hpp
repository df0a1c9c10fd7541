// Masking of a row's last chain for the pipelined row streams
// (rows_kernels.hip, rows_fixed_kernels.hip).
#pragma once

#include "device_common.hpp"

namespace armx {
namespace dev {

// The masks of a row's last chain.  Every row has the same cols, so the
// selection mask_row_chain makes in the last chain is the same for every row:
// keep[r] holds all bits for the values of chunk r of that chain that lie in
// the row and none for the others, computed once per wavefront, and
// apply_row_tail then costs one bitwise select per register (the per-chain
// computation of mask_row_chain, repeated for every row, kept one wavefront
// per SIMD busy long enough to halve the row stream's throughput).
template <int R>
__device__ __forceinline__ void row_tail_keep(uint64_t cols, int lane, u32x4 (&keep)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) keep[r] = u32x4{~0u, ~0u, ~0u, ~0u};
  mask_row_chain<R>(keep, (cols - 1) / (uint64_t(R) * 512), cols, 0u, lane);
}

// v = v where keep is set, else `fill` (a binary16 pattern): the last chain
// of a row masked as mask_row_chain would mask it.
template <int R>
__device__ __forceinline__ void apply_row_tail(u32x4 (&v)[R], const u32x4 (&keep)[R],
                                               uint32_t fill) {
  const uint32_t f2 = fill | (fill << 16);
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int w = 0; w < 4; ++w) v[r][w] = (v[r][w] & keep[r][w]) | (f2 & ~keep[r][w]);
  }
}

}  // namespace dev
}  // namespace armx
