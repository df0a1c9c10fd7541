// Row-segmented sum: out[r] = sum of x[r * ld + c] over c < cols.
//
// Many independent sums of the kind in "GPU Tensor Cores for fast Arithmetic
// Reductions" (arXiv 2001.05585), Abstract, one per row.  Every chunk of a
// row goes through one v_mfma_f32_16x16x32_f16 against the signed ones
// operand (or all ones with ARMX_FLAG_ALL_ONES; or, with ARMX_FLAG_PLAIN,
// per-lane fp32 adds; the designs of device_common.hpp) and R of them chain
// into the fp32 accumulators.  A chunk never straddles two rows: the chunk
// grid restarts at every row (rows are 16-byte aligned because ld is a
// multiple of 8), and a row's last partial chain is masked.  Rows of at most 512 values go to
// the segmented kernel of short_rows_kernels.hip instead.  The row's fp32
// total is written directly, except in the split mapping, where a row's parts
// meet in a workspace and the last block adds them.  The mappings:
//  * wave_rows: each wavefront sums whole rows (rows g, g + T, ... for
//    wavefront g of T); the loads of the next row are issued before the
//    current row is finished, so the pipeline runs across rows, and a row's
//    last partial chain is masked in registers (the matrix's last row then
//    takes exact masked loads instead); no block synchronisation at all.
//    Used when there are many rows; rows of at least kRowsLongMinCols values
//    run rows_stream_kernel, which keeps the last row in the stream and reads
//    only its last chain apart.
//  * rows_split_kernel (few rows, or a row stream whose last round would be
//    poorly filled; with a workspace): every row is split over S wavefronts
//    of several blocks, which take the row's chains round-robin as the flat
//    sum's wavefronts take the input's, each with its own paced pipeline;
//    each publishes its partial, and the last block to finish writes every
//    row's balanced tree over its S partials.
//  * otherwise each block sums a row (looping over rows if needed) and its W
//    wavefronts take the row's chains round-robin, combined through LDS.
#include "device_common.hpp"
#include "row_tail.hpp"
#include "launch.h"

namespace armx {
namespace {

using namespace dev;

// Position in this wavefront's sequence of (row, chain) items: rows
// g, g + T, g + 2T, ... (k counts them) and chains 0 .. cpr-1 of each.
struct RowCursor {
  uint64_t k = 0, c = 0;
  __device__ __forceinline__ void next(uint64_t cpr) {
    if (++c == cpr) {
      c = 0;
      ++k;
    }
  }
};

// The flattened stream of one wavefront's rows (rows g, g + T, ... below
// `rows`, which must not include the matrix's last row when rows end inside
// a chain): loads run ahead across row boundaries, so the pipeline never
// drains between rows.  A row that is not a whole number of chains ends in a
// partial chain, read and masked as load_row_chain and mask_row_chain
// describe (values past the row count as +0.0; the masks are computed once,
// by row_tail_keep).  At the end of a row its total is written and the
// running sum restarts.
// PARTIAL: whether rows end inside a chain (instantiated apart, so that whole
// chains carry no masking code at all).  RANGE (with PARTIAL, for rows of
// less than 2 GiB): the chains are read by load_row_chain_range, so nothing
// past a row's last 16-byte slot is fetched.
template <int R, bool NT, int D, bool PARTIAL, bool RANGE = false>
__device__ __forceinline__ void rows_flat(const uint16_t* __restrict__ x, uint64_t rows,
                                          uint64_t cols, uint64_t ld, float* __restrict__ out,
                                          uint64_t g, uint64_t T, int lane) {
  if (g >= rows) return;
  const uint64_t chain_elems = uint64_t(R) * 512;
  const uint64_t cpr = (cols + chain_elems - 1) / chain_elems;
  const uint64_t last_chunk = (cols - 1) / 512;
  const u32x4* fill = neg_zero_chunk();
  const uint32_t row_bytes = uint32_t((cols * 2 + 15) & ~uint64_t(15));
  u32x4 keep[R];
  if constexpr (PARTIAL) row_tail_keep<R>(cols, lane, keep);
  const uint64_t K = (rows - 1 - g) / T + 1;
  const uint64_t items = K * cpr;
  const uint64_t row_step = T * ld;
  RowCursor pf, rd, pr;   // next item to load, to reduce, to retire
  const uint16_t* load_row = x + g * ld;
  auto load = [&](u32x4 (&v)[R]) {
    if constexpr (RANGE) {
      load_row_chain_range<R, NT>(load_row, row_bytes, pf.c, lane, v);
    } else {
      load_row_chain<R, NT>(load_row, pf.c, last_chunk, fill, lane, v);
    }
    // stays on the last item once it is reached (the re-read is not used)
    if (pf.c + 1 < cpr) {
      ++pf.c;
    } else if (pf.k + 1 < K) {
      pf.c = 0;
      ++pf.k;
      load_row += row_step;
    }
  };
  // A chain's value joins the running sum one half-step later (after the next
  // loads are issued), so waiting for it never delays a prefetch.
  float run = 0.0f, pending = 0.0f;
  bool have_pending = false;
  auto retire = [&]() {
    if (!have_pending) return;
    run += pending;
    have_pending = false;
    if (pr.c + 1 == cpr) {
      const float total = wave_total<D>(run);
      if (lane == 0) out[g + pr.k * T] = total;
      run = 0.0f;
    }
    pr.next(cpr);
  };
  auto reduce = [&](u32x4 (&v)[R]) {
    retire();
    if constexpr (PARTIAL) {
      if (rd.c + 1 == cpr) apply_row_tail<R>(v, keep, 0u);
    }
    pending = chain_value<R, D>(v);
    have_pending = true;
    rd.next(cpr);
  };
  u32x4 a[R], b[R];
  load(a);
  for (uint64_t j = 0; j < items; j += 2) {
    load(b);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the tile steps
    reduce(a);
    load(a);
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 < items) reduce(b);
  }
  retire();
}

// One row summed by one wavefront with exact masked loads (no read past
// the row): its whole chains pipelined, then the partial chain.
template <int R, bool NT, int D>
__device__ __forceinline__ float row_total_masked(const uint16_t* __restrict__ xr, uint64_t cols,
                                                  int lane) {
  const uint64_t chains_full = cols / (uint64_t(R) * 512);
  float run = 0.0f;
  stream_chains<R, NT, D>(reinterpret_cast<const u32x4*>(xr), 0, chains_full, 1, lane, run);
  if (chains_full * R * 512 < cols) tail_chain<R, D>(xr, chains_full, cols, lane, run);
  return wave_total<D>(run);
}

// rows_flat for long rows: the same stream, but the matrix's last row stays
// in it (the owner wavefront streams all of its rows), and only that row's
// last chain, whose pipelined loads would read on past the matrix, is read
// apart after the stream with load_last_chain (nothing past the row).  On
// few long rows the last row summed apart by its owner finished well after
// the others (1000 rows of 268288 values: 107 us against 85 us streamed);
// on rows under 64 chunks this form measured up to 3 us slower than
// rows_flat (67243 rows of 3992 values: 80.5 against 77.3 us), so the
// launch takes it from 32768 values per row on.
template <int R, bool NT, int D, bool PARTIAL>
__device__ __forceinline__ void rows_flat_long(const uint16_t* __restrict__ x, uint64_t rows,
                                               uint64_t cols, uint64_t ld,
                                               float* __restrict__ out, uint64_t g, uint64_t T,
                                               int lane) {
  if (g >= rows) return;
  const uint64_t chain_elems = uint64_t(R) * 512;
  const uint64_t cpr = (cols + chain_elems - 1) / chain_elems;
  const uint64_t last_chunk = (cols - 1) / 512;
  const u32x4* fill = neg_zero_chunk();
  u32x4 keep[R];
  if constexpr (PARTIAL) row_tail_keep<R>(cols, lane, keep);
  const uint64_t K = (rows - 1 - g) / T + 1;
  const bool last_apart = PARTIAL && g + (K - 1) * T == rows - 1;
  // streamed (row, chain) items: fewer than 2^32 (the matrix holds at most
  // 2^40 values, and every chain but a row's last holds 4096)
  const uint32_t items = uint32_t(K * cpr - (last_apart ? 1 : 0));
  const uint64_t row_step = T * ld;
  RowCursor rd, pr;   // next item to reduce, to retire
  uint64_t lc = 0;    // chain of the next item to load
  uint32_t issued = 0;
  const uint16_t* load_row = x + g * ld;
  auto load = [&](u32x4 (&v)[R]) {
    load_row_chain_counted<R, NT, PARTIAL>(load_row, lc, last_chunk, fill, lane, v);
    // stays on the last streamed item once it is reached (the re-read is not used)
    if (++issued < items) {
      if (lc + 1 < cpr) {
        ++lc;
      } else {
        lc = 0;
        load_row += row_step;
      }
    }
  };
  // A chain's value joins the running sum one half-step later (after the next
  // loads are issued), so waiting for it never delays a prefetch.
  float run = 0.0f, pending = 0.0f;
  bool have_pending = false;
  auto retire = [&]() {
    if (!have_pending) return;
    run += pending;
    have_pending = false;
    if (pr.c + 1 == cpr) {
      const float total = wave_total<D>(run);
      if (lane == 0) out[g + pr.k * T] = total;
      run = 0.0f;
    }
    pr.next(cpr);
  };
  auto reduce = [&](u32x4 (&v)[R]) {
    retire();
    if constexpr (PARTIAL) {
      if (rd.c + 1 == cpr) apply_row_tail<R>(v, keep, 0u);
    }
    pending = chain_value<R, D>(v);
    have_pending = true;
    rd.next(cpr);
  };
  if (items > 0) {
    u32x4 a[R], b[R];
    load(a);
    for (uint32_t j = 0; j < items; j += 2) {
      load(b);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the tile steps
      reduce(a);
      load(a);
      __builtin_amdgcn_sched_barrier(0);
      if (j + 1 < items) reduce(b);
    }
    retire();
  }
  if constexpr (PARTIAL) {
    if (last_apart) {
      u32x4 fin[R];
      uint32_t fin_h[8];
      load_last_chain<R, NT>(x + (rows - 1) * ld, cpr - 1, cols, lane, fin, fin_h);
      merge_last_chain<R>(fin, fin_h, cpr - 1, cols, lane);
      apply_row_tail<R>(fin, keep, 0u);
      run += chain_value<R, D>(fin);
      const float total = wave_total<D>(run);
      if (lane == 0) out[rows - 1] = total;
    }
  }
}

// The wave_rows mapping for rows of at least kRowsLongMinCols values, with
// rows_flat_long, as a kernel of its own for blocks of at most
// kRowsStreamMaxBlock threads (compiled for such blocks, a wavefront may hold
// more than the 128 registers a 1024-thread block leaves, and at R = 8 it
// needs them: rows_kernel spills there).
template <int R, bool NT, int D>
__global__ __launch_bounds__(kRowsStreamMaxBlock) void rows_stream_kernel(
    const uint16_t* __restrict__ x, uint64_t rows, uint64_t cols, uint64_t ld,
    float* __restrict__ out, int remap) {
  const int lane = lane_id();
  const uint64_t W = uint64_t(num_waves());
  const uint64_t g = (remap ? xcd_block_id() : uint64_t(blockIdx.x)) * W + uint64_t(wave_id());
  const uint64_t T = uint64_t(gridDim.x) * W;
  if (cols % (uint64_t(R) * 512) != 0) {
    rows_flat_long<R, NT, D, true>(x, rows, cols, ld, out, g, T, lane);
  } else {
    rows_flat_long<R, NT, D, false>(x, rows, cols, ld, out, g, T, lane);
  }
}

template <int R, bool NT, int D>
__global__ __launch_bounds__(1024) void rows_kernel(const uint16_t* __restrict__ x, uint64_t rows,
                                                    uint64_t cols, uint64_t ld,
                                                    float* __restrict__ out, int wave_rows,
                                                    int remap) {
  __shared__ float red[16];
  const int lane = lane_id();
  const uint64_t W = uint64_t(num_waves());
  const uint64_t chains_full = cols / (uint64_t(R) * 512);
  const bool tail = chains_full * R * 512 < cols;

  if (wave_rows) {
    const uint64_t g = (remap ? xcd_block_id() : uint64_t(blockIdx.x)) * W + uint64_t(wave_id());
    const uint64_t T = uint64_t(gridDim.x) * W;
    // the last row stays out of the stream when rows end inside a chain
    const uint64_t streamed = tail ? rows - 1 : rows;
    if (tail && cols < kRowsRangeMaxCols) {
      rows_flat<R, NT, D, true, true>(x, streamed, cols, ld, out, g, T, lane);
    } else if (tail) {
      rows_flat<R, NT, D, true>(x, streamed, cols, ld, out, g, T, lane);
    } else {
      rows_flat<R, NT, D, false>(x, streamed, cols, ld, out, g, T, lane);
    }
    if (tail && g == (rows - 1) % T) {
      const float total = row_total_masked<R, NT, D>(x + (rows - 1) * ld, cols, lane);
      if (lane == 0) out[rows - 1] = total;
    }
    return;
  }

  for (uint64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const uint16_t* xr = x + row * ld;
    float run = 0.0f;
    const uint64_t c = uint64_t(wave_id());
    const uint64_t iters = c < chains_full ? (chains_full - 1 - c) / W + 1 : 0;
    stream_chains<R, NT, D>(reinterpret_cast<const u32x4*>(xr), c, iters, W, lane, run);
    if (tail && c + iters * W == chains_full) tail_chain<R, D>(xr, chains_full, cols, lane, run);
    const float total = block_sum_lane0(wave_total<D>(run), red);
    if (threadIdx.x == 0) out[row] = total;
  }
}

// Few rows: wavefront `item` (block * W + wave) is segment s = item % S of row
// item / S and takes that row's chains s, s + S, ...; the row's partial
// chain (if any) goes to the wavefront whose turn it is, with exact masked
// loads.  Partials go to partials[item]; one completion counter, and the last
// block writes out[r] = the balanced tree over row r's S partials in index
// order (combine_split_rows), so the result depends on the configuration
// only.
template <int R, bool NT, int D>
__global__ __launch_bounds__(1024) void rows_split_kernel(const uint16_t* __restrict__ x,
                                                          uint64_t rows, uint64_t cols,
                                                          uint64_t ld, float* __restrict__ out,
                                                          unsigned segs,
                                                          unsigned* __restrict__ counter,
                                                          float* __restrict__ partials) {
  __shared__ int flag;
  __shared__ float stage[kSplitMaxItems];
  const int lane = lane_id();
  const uint64_t W = uint64_t(num_waves());
  const uint64_t S = segs;
  const uint64_t item = uint64_t(blockIdx.x) * W + uint64_t(wave_id());
  if (item < rows * S) {
    const uint64_t row = item / S, s = item % S;
    const uint16_t* xr = x + row * ld;
    const u32x4* xv = reinterpret_cast<const u32x4*>(xr);
    const uint64_t chains_full = cols / (uint64_t(R) * 512);
    const uint64_t iters = s < chains_full ? (chains_full - 1 - s) / S + 1 : 0;
    float run = 0.0f;
    // pacing as for the flat sum
    if (iters >= kPaceLongChains) {
      stream_chains<R, NT, D, D == kPlain ? 4 : 8>(xv, s, iters, S, lane, run);
    } else if (D != kPlain && iters >= kPaceShortChains) {
      stream_chains<R, NT, D, 2>(xv, s, iters, S, lane, run);
    } else {
      stream_chains<R, NT, D>(xv, s, iters, S, lane, run);
    }
    if (chains_full * R * 512 < cols && s + iters * S == chains_full)
      tail_chain<R, D>(xr, chains_full, cols, lane, run);
    const float total = wave_total<D>(run);
    if (lane == 0) __hip_atomic_store(partials + item, total, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial is stored
  }
  __syncthreads();   // every wavefront's partial is stored before the block counts
  if (!publish_with_ticket([] {}, counter, gridDim.x, &flag)) return;
  combine_split_rows(partials, rows, segs, out, stage, unsigned(W) * 64);
}

template <template <int, bool, int> class K, int R, bool NT>
const void* pick_design(int d) {
  switch (d) {
    case kSigned: return K<R, NT, kSigned>::ptr();
    case kPlain: return K<R, NT, kPlain>::ptr();
    case kOnes: return K<R, NT, kOnes>::ptr();
    default: return nullptr;
  }
}

template <template <int, bool, int> class K, int R>
const void* pick_nt(bool nt, int d) {
  return nt ? pick_design<K, R, true>(d) : pick_design<K, R, false>(d);
}

template <template <int, bool, int> class K>
const void* kernel_for(int r, bool nt, int d) {
  switch (r) {
    case 1: return pick_nt<K, 1>(nt, d);
    case 2: return pick_nt<K, 2>(nt, d);
    case 3: return pick_nt<K, 3>(nt, d);
    case 4: return pick_nt<K, 4>(nt, d);
    case 5: return pick_nt<K, 5>(nt, d);
    case 6: return pick_nt<K, 6>(nt, d);
    case 7: return pick_nt<K, 7>(nt, d);
    case 8: return pick_nt<K, 8>(nt, d);
    default: return nullptr;
  }
}

template <int R, bool NT, int D>
struct RowsK {
  static const void* ptr() { return reinterpret_cast<const void*>(&rows_kernel<R, NT, D>); }
};

template <int R, bool NT, int D>
struct StreamK {
  static const void* ptr() {
    return reinterpret_cast<const void*>(&rows_stream_kernel<R, NT, D>);
  }
};

template <int R, bool NT, int D>
struct SplitK {
  static const void* ptr() {
    return reinterpret_cast<const void*>(&rows_split_kernel<R, NT, D>);
  }
};

}  // namespace

hipError_t launch_rows(const Plan& plan, const void* x, float* out, void* ws,
                       hipStream_t stream) {
  if (plan.rows == 0) return hipSuccess;
  if (plan.n == 0) return launch_zero(out, plan.rows, stream);
  if (plan.mode == 2) return launch_short_rows(plan, x, out, stream);
  if (plan.mode == 3) {
    const void* fn = kernel_for<SplitK>(plan.r, (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0,
                                        chain_design(plan.flags));
    if (!fn || !ws || plan.segs > kSplitMaxSegs || plan.rows * plan.segs > kSplitMaxItems)
      return hipErrorInvalidValue;   // more parts than the last block's stage and tree hold
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    uint64_t rows = plan.rows, cols = plan.n, ld = plan.ld;
    unsigned segs = plan.segs;
    Workspace w = workspace_layout(plan, ws);
    void* args[] = {&xh, &rows, &cols, &ld, &out, &segs, &w.counters, &w.partials};
    return launch_main(plan, fn, args, stream);
  }
  const bool nt = (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0;
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  uint64_t rows = plan.rows, cols = plan.n, ld = plan.ld;
  int wave_rows = plan.mode;
  int remap = plan.xcd_remap;
  if (wave_rows && cols >= kRowsLongMinCols && plan.waves * 64 <= kRowsStreamMaxBlock) {
    const void* fn = kernel_for<StreamK>(plan.r, nt, chain_design(plan.flags));
    if (!fn) return hipErrorInvalidValue;
    void* args[] = {&xh, &rows, &cols, &ld, &out, &remap};
    return launch_main(plan, fn, args, stream);
  }
  const void* fn = kernel_for<RowsK>(plan.r, nt, chain_design(plan.flags));
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {&xh, &rows, &cols, &ld, &out, &wave_rows, &remap};
  return launch_main(plan, fn, args, stream);
}

}  // namespace armx
