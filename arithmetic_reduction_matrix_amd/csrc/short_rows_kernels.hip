// Row sums of rows no longer than one chunk (cols <= 512), for both row
// entry points.
//
// A row of cols values takes P = 2^S lanes, the power of two at or above
// ceil(cols / 8), one 16-byte slot of 8 values each; a wavefront load then
// covers a group of 64 / P rows, and a wavefront takes G groups per step (8,
// or 4 for rows of more than 32 values at a pitch of whole 128-byte lines).
// The chunk grid of the longer-row kernels would give every such row a whole
// 512-value load of its own, mostly masked; here every lane of every load
// carries data whenever cols fills its P slots.
//
// Each lane's 8 values are levels 1-3 of the row's balanced tree (the leaves
// widened exactly to binary32, padded with -0.0, every node one binary32
// round-to-nearest-even addition: "Taming Bitwise Behavior in GPU Kernels with
// Tensor Core", arXiv 2609.11356, Abstract), and the row's P lanes are levels
// 4 to 3 + S by the lane ladder, so every lane of a row ends with the row's
// root.  The result is the row's fixed-order sum, which is also a valid
// free-order sum: the all-ones MFMA of "GPU Tensor Cores for fast Arithmetic
// Reductions" (arXiv 2001.05585, Abstract) adds values of lanes 16 apart,
// which here belong to different rows, so one MFMA per load cannot serve.
//
// With MMA (the order with MFMA leaves, for the fixed-order entry point) a
// row's node is instead the one its 512-value chunk has in that order: one
// v_mfma_f32_16x16x32_f16 against ones from a zero accumulator, column j
// summing the row's slots j, j + 16, j + 32, j + 48 in that K order, and the
// balanced tree over the 16 column sums.  Since lanes 16 apart feed the same
// MFMA column, every block of max(16, P) lanes gets an MFMA of its own with
// the other lanes' values zeroed (short_row_node_mma).
//
// Output: rows of more than 32 values (short_rows_staged_kernel) are cut into
// chunks of consecutive rows (at most kShortChunkRows); a block reduces a
// chunk with all its wavefronts, keeps the row sums in LDS, and writes the
// chunk's sums out with consecutive 4-byte stores when every wavefront is
// done, so the output leaves the compute units in bursts rather than a few
// bytes per wavefront step between the loads.  Narrower rows
// (short_rows_direct_kernel), whose sums are too many for that, are stored as
// they are reduced, by wavefronts that take the steps of the whole matrix in
// turn.
//
// The loop body has no branches.  Every load is unconditional: a lane past
// the row's last slot reads the last slot again, a row past the end (of the
// matrix, or of the chunk) reads the last row again, and values that are not
// the row's are replaced by -0.0 with per-lane masks.  Those re-read rows are
// reduced like the real ones and write the same value to the same place.  A
// slot that straddles the end of the row reads 16 bytes of which the tail
// lies in the row's pitch (ld is a multiple of 8 when there is more than one
// row); only the last row of a matrix whose cols is not a multiple of 8 could
// end inside such a slot, so that row is summed apart, with element loads.
#include "fixed_tree.hpp"
#include "launch.h"

namespace armx {
namespace {

using namespace dev;
using namespace dev::tree;

constexpr uint32_t kNegZero2 = 0x80008000u;

// Levels 1-3 of the tree over one lane's 8 values.
__device__ __forceinline__ float leaf8(u32x4 t) {
  const float b0 = pair_node(t[0]) + pair_node(t[1]);
  const float b1 = pair_node(t[2]) + pair_node(t[3]);
  return b0 + b1;
}

// A row's node in the order with MFMA leaves, for rows of P = 2^S lanes
// packed 64 / P to a load (lane i of a row is its slot i).  Lane blocks of
// 2^B = max(16, P) lanes each take one MFMA against ones from a zero
// accumulator, with every lane outside the block zeroed.  The K positions of
// such an MFMA that hold zeros leave the zero accumulator as it is, and the
// block's slots sit in K order (slot i of a P = 32 row in the upper half at K
// group 2 + i / 16), so each column sum is the one the row's own chunk gives.
// Lane l then holds column l % 16 of its block: its own column.  The tree over
// the row's 16 columns follows: for P < 16 the columns past the row's slots
// are +0.0 sums and form subtrees of +0.0, which leave a node that is not
// -0.0 unchanged (no MFMA from a zero accumulator returns -0.0), so the tree
// over the row's P lanes is the node; for P = 32 the two 16-lane halves hold
// the same columns and each finishes the tree alone.
template <int S>
__device__ __forceinline__ float short_row_node_mma(u32x4 t, int lane) {
  constexpr int B = S < 4 ? 4 : S;
  constexpr int NB = 64 >> B;
  const int blk = lane >> B;
  float own = 0.0f;
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    u32x4 tq;
#pragma unroll
    for (int w = 0; w < 4; ++w) tq[w] = blk == q ? t[w] : 0u;
    const float c = mfma_ones(floatx4{0.0f, 0.0f, 0.0f, 0.0f}, tq)[0];
    own = blk == q ? c : own;
  }
  return lane_tree(own, S < 4 ? S : 4);
}

template <int S, bool MMA>
__device__ __forceinline__ float short_row_node(u32x4 t, int lane) {
  if constexpr (MMA) {
    return short_row_node_mma<S>(t, lane);
  } else {
    return lane_tree(leaf8(t), S);
  }
}

// The same nodes from one MFMA per load: the A operand, all ones in
// short_row_node_mma, becomes a selector with A[i][k] = 1 when K position k
// belongs to the lane block whose lanes receive output row i (lane l holds
// output rows 4 (l / 16) .. + 3 of column l % 16), else 0.  Every output row
// then sums only its own block's K groups, the others contributing zero
// products, so every lane again ends with its own column sum.  A lane
// supplies A[l % 16][8 (l / 16) .. + 7]: one value for all eight.  Only for
// finite inputs: 0 x Inf is NaN, which would reach the other blocks' rows in
// that column (the caller checks).
template <int S>
__device__ __forceinline__ half8 block_selector(int lane) {
  constexpr int B = S < 4 ? 4 : S;
  const bool on = ((lane >> 4) >> (B - 4)) == (((lane & 15) >> 2) >> (B - 4));
  const _Float16 v = on ? _Float16(1.0f) : _Float16(0.0f);
  return half8{v, v, v, v, v, v, v, v};
}

template <int S>
__device__ __forceinline__ float short_row_node_sel(u32x4 t, half8 sel) {
  const floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(
      sel, __builtin_bit_cast(half8, t), floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
  return lane_tree(c[0], S < 4 ? S : 4);
}

// Whether any of this lane's 8 values is an Inf or a NaN (exponent field all
// ones): the largest masked exponent field of each half-word column.
__device__ __forceinline__ bool has_non_finite(u32x4 t) {
  using u16x2 = unsigned short __attribute__((ext_vector_type(2)));
  constexpr uint32_t kExp = 0x7C007C00u;
  u16x2 m = __builtin_bit_cast(u16x2, t[0] & kExp);
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, t[1] & kExp));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, t[2] & kExp));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, t[3] & kExp));
  return (m[0] == 0x7C00u) | (m[1] == 0x7C00u);
}

// Rows of at most 32 values (S <= 2): every wavefront of the grid takes the
// steps in turn and stores its rows' sums as it goes, 8 groups per step.
template <int S, bool NT, bool MMA>
__global__ __launch_bounds__(MMA ? kShortMmaMaxBlock : 1024) void short_rows_direct_kernel(
    const uint16_t* __restrict__ x, uint64_t rows, uint64_t cols, uint64_t ld,
    float* __restrict__ out, int remap) {
  constexpr uint64_t P = uint64_t(1) << S;
  constexpr int G = 8;
  constexpr uint64_t RPG = 64 >> S;   // rows per group (one wavefront load)
  constexpr uint64_t RPS = RPG * G;   // rows per step
  const int lane = lane_id();
  const uint64_t W = uint64_t(num_waves());
  const uint64_t g = (remap ? xcd_block_id() : uint64_t(blockIdx.x)) * W + uint64_t(wave_id());
  const uint64_t T = uint64_t(gridDim.x) * W;
  const uint64_t slot = uint64_t(lane) & (P - 1);
  const uint64_t sub = uint64_t(lane) >> S;
  const uint64_t last_slot = (cols - 1) / 8;
  const uint64_t read_slot = slot < last_slot ? slot : last_slot;

  // halves of this lane's slot that hold the row's values
  const uint64_t e = slot * 8;
  const uint64_t k = e >= cols ? 0 : (cols - e >= 8 ? 8 : cols - e);
  u32x4 keep;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    keep[w] = (uint64_t(2 * w) < k ? 0xFFFFu : 0u) | (uint64_t(2 * w + 1) < k ? 0xFFFF0000u : 0u);

  const bool ragged = (cols % 8) != 0;
  const uint64_t body = ragged ? rows - 1 : rows;   // rows read with whole slots
  if (ragged && g == T - 1) {
    const uint16_t* xr = x + (rows - 1) * ld;
    const float root = short_row_node<S, MMA>(load8_clamped(xr, e, cols, 0x8000u), lane);
    if (lane == 0) out[rows - 1] = root;
  }

  const uint64_t steps = (body + RPS - 1) / RPS;
  if (g >= steps) return;
  const uint64_t K = (steps - 1 - g) / T + 1;   // this wavefront's steps
  auto row_of = [&](uint64_t c, int u) {
    const uint64_t r = c * RPS + uint64_t(u) * RPG + sub;
    return r < body ? r : body - 1;
  };
  auto load_step = [&](uint64_t c, u32x4 (&v)[G]) {
#pragma unroll
    for (int u = 0; u < G; ++u)
      v[u] = load16<NT>(reinterpret_cast<const u32x4*>(x + row_of(c, u) * ld) + read_slot);
  };
  const half8 sel = block_selector<S>(lane);
  // values that are not the row's become -0.0
  auto row_values = [&](const u32x4& v) {
    u32x4 t;
#pragma unroll
    for (int w = 0; w < 4; ++w) t[w] = (v[w] & keep[w]) | (kNegZero2 & ~keep[w]);
    return t;
  };
  auto reduce_step = [&](uint64_t c, const u32x4 (&v)[G]) {
    if constexpr (!MMA) {
#pragma unroll
      for (int u = 0; u < G; ++u)   // the same value in every lane of the row
        out[row_of(c, u)] = lane_tree(leaf8(row_values(v[u])), S);
    } else {
      u32x4 t[G];
#pragma unroll
      for (int u = 0; u < G; ++u) t[u] = row_values(v[u]);
      // one selector MFMA per load unless the step holds an Inf or a NaN (then
      // a masked MFMA per lane block); one row per load (P = 64) needs neither
      bool one_mfma = true;
      if constexpr (S < 6) {
        bool nf = false;
#pragma unroll
        for (int u = 0; u < G; ++u) nf = nf | has_non_finite(t[u]);
        one_mfma = __builtin_amdgcn_ballot_w64(nf) == 0;
      }
      // no memory access inside the branch: stores there make the compiler
      // wait for every load in flight where the two paths join
      float node[G];
      if (one_mfma) {
#pragma unroll
        for (int u = 0; u < G; ++u) node[u] = short_row_node_sel<S>(t[u], sel);
      } else {
#pragma unroll
        for (int u = 0; u < G; ++u) node[u] = short_row_node_mma<S>(t[u], lane);
      }
#pragma unroll
      for (int u = 0; u < G; ++u) out[row_of(c, u)] = node[u];
    }
  };
  auto step = [&](uint64_t j) { return g + (j < K ? j : K - 1) * T; };

  // Software pipeline with ping-pong buffers, as in the flat kernels: the next
  // step's loads are issued before the current step is reduced; past the last
  // step the loads and the reduction repeat it.
  u32x4 a[G], b[G];
  load_step(step(0), a);
  for (uint64_t j = 0; j < K; j += 2) {
    load_step(step(j + 1), b);
    __builtin_amdgcn_sched_barrier(0);
    reduce_step(step(j), a);
    load_step(step(j + 2), a);
    __builtin_amdgcn_sched_barrier(0);
    reduce_step(step(j + 1), b);
  }
}

// Rows of more than 32 values (S >= 3): chunks of rows staged in LDS.
template <int S, int G, bool NT, bool MMA>
__global__ __launch_bounds__(MMA ? kShortMmaMaxBlock : 1024) void short_rows_staged_kernel(
    const uint16_t* __restrict__ x, uint64_t rows, uint64_t cols, uint64_t ld,
    float* __restrict__ out, uint64_t chunk_rows) {
  extern __shared__ float staged[];   // the chunk's sums (chunk_rows floats)
  constexpr uint64_t P = uint64_t(1) << S;
  constexpr uint64_t RPG = 64 >> S;   // rows per group (one wavefront load)
  constexpr uint64_t RPS = RPG * G;   // rows per step
  const int lane = lane_id();
  const uint64_t W = uint64_t(num_waves());
  const uint64_t w = uint64_t(wave_id());
  const uint64_t bid = blockIdx.x;   // a chunk is one block's range of rows
  const uint64_t slot = uint64_t(lane) & (P - 1);
  const uint64_t sub = uint64_t(lane) >> S;
  const uint64_t last_slot = (cols - 1) / 8;
  const uint64_t read_slot = slot < last_slot ? slot : last_slot;

  // halves of this lane's slot that hold the row's values
  const uint64_t e = slot * 8;
  const uint64_t k = e >= cols ? 0 : (cols - e >= 8 ? 8 : cols - e);
  u32x4 keep;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    keep[q] = (uint64_t(2 * q) < k ? 0xFFFFu : 0u) | (uint64_t(2 * q + 1) < k ? 0xFFFF0000u : 0u);

  const bool ragged = (cols % 8) != 0;
  const uint64_t body = ragged ? rows - 1 : rows;   // rows read with whole slots
  if (ragged && bid == gridDim.x - 1 && w == W - 1) {
    const uint16_t* xr = x + (rows - 1) * ld;
    const float root = short_row_node<S, MMA>(load8_clamped(xr, e, cols, 0x8000u), lane);
    if (lane == 0) out[rows - 1] = root;
  }

  const half8 sel = block_selector<S>(lane);
  // values that are not the row's become -0.0
  auto row_values = [&](const u32x4& v) {
    u32x4 t;
#pragma unroll
    for (int q = 0; q < 4; ++q) t[q] = (v[q] & keep[q]) | (kNegZero2 & ~keep[q]);
    return t;
  };

  // Rows [r0, r1) in steps of RPS rows; this wavefront takes steps first,
  // first + stride, ... and puts every row's sum in LDS at its place in the
  // chunk.  A row past r1 reads and sums row r1 - 1 again.
  auto stream = [&](uint64_t r0, uint64_t r1, uint64_t first, uint64_t stride) {
    const uint64_t steps = (r1 - r0 + RPS - 1) / RPS;
    if (first >= steps) return;
    const uint64_t K = (steps - 1 - first) / stride + 1;   // this wavefront's steps
    auto row_of = [&](uint64_t c, int u) {
      const uint64_t r = r0 + c * RPS + uint64_t(u) * RPG + sub;
      return r < r1 ? r : r1 - 1;
    };
    auto load_step = [&](uint64_t c, u32x4 (&v)[G]) {
#pragma unroll
      for (int u = 0; u < G; ++u)
        v[u] = load16<NT>(reinterpret_cast<const u32x4*>(x + row_of(c, u) * ld) + read_slot);
    };
    auto reduce_step = [&](uint64_t c, const u32x4 (&v)[G]) {
      float node[G];
      if constexpr (!MMA) {
#pragma unroll
        for (int u = 0; u < G; ++u)   // the same value in every lane of the row
          node[u] = lane_tree(leaf8(row_values(v[u])), S);
      } else {
        u32x4 t[G];
#pragma unroll
        for (int u = 0; u < G; ++u) t[u] = row_values(v[u]);
        // one selector MFMA per load unless the step holds an Inf or a NaN
        // (then a masked MFMA per lane block); one row per load (P = 64)
        // needs neither
        bool one_mfma = true;
        if constexpr (S < 6) {
          bool nf = false;
#pragma unroll
          for (int u = 0; u < G; ++u) nf = nf | has_non_finite(t[u]);
          one_mfma = __builtin_amdgcn_ballot_w64(nf) == 0;
        }
        // no memory access inside the branch: stores there make the compiler
        // wait for every load in flight where the two paths join
        if (one_mfma) {
#pragma unroll
          for (int u = 0; u < G; ++u) node[u] = short_row_node_sel<S>(t[u], sel);
        } else {
#pragma unroll
          for (int u = 0; u < G; ++u) node[u] = short_row_node_mma<S>(t[u], lane);
        }
      }
      if (slot == 0) {
#pragma unroll
        for (int u = 0; u < G; ++u) staged[row_of(c, u) - r0] = node[u];
      }
    };
    auto step = [&](uint64_t j) { return first + (j < K ? j : K - 1) * stride; };

    // Software pipeline with ping-pong buffers, as in the flat kernels: the
    // next step's loads are issued before the current step is reduced; past
    // the last step the loads and the reduction repeat it.
    u32x4 a[G], b[G];
    load_step(step(0), a);
    for (uint64_t j = 0; j < K; j += 2) {
      load_step(step(j + 1), b);
      __builtin_amdgcn_sched_barrier(0);
      reduce_step(step(j), a);
      load_step(step(j + 2), a);
      __builtin_amdgcn_sched_barrier(0);
      reduce_step(step(j + 1), b);
    }
  };

  // Chunks of consecutive rows, taken by the blocks in turn; the block's
  // wavefronts take the chunk's steps in turn, one lane of each row puts its
  // sum in LDS, and the block writes the chunk's sums out together once every
  // wavefront is done with it.
  const uint64_t chunks = (body + chunk_rows - 1) / chunk_rows;
  for (uint64_t ch = bid; ch < chunks; ch += gridDim.x) {
    const uint64_t r0 = ch * chunk_rows;
    const uint64_t r1 = r0 + chunk_rows < body ? r0 + chunk_rows : body;
    stream(r0, r1, w, W);
    __syncthreads();
    // 8 LDS reads in flight per thread before their stores
    const uint64_t cnt = r1 - r0, T = blockDim.x;
    uint64_t i = threadIdx.x;
    for (; i + 7 * T < cnt; i += 8 * T) {
      float t[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) t[q] = staged[i + uint64_t(q) * T];
#pragma unroll
      for (int q = 0; q < 8; ++q) out[r0 + i + uint64_t(q) * T] = t[q];
    }
    for (; i < cnt; i += T) out[r0 + i] = staged[i];
    __syncthreads();   // the next chunk reuses the LDS
  }
}

template <int S>
const void* pick_direct(bool nt, bool mma) {
  if (mma)
    return nt ? reinterpret_cast<const void*>(&short_rows_direct_kernel<S, true, true>)
              : reinterpret_cast<const void*>(&short_rows_direct_kernel<S, false, true>);
  return nt ? reinterpret_cast<const void*>(&short_rows_direct_kernel<S, true, false>)
            : reinterpret_cast<const void*>(&short_rows_direct_kernel<S, false, false>);
}

template <int S, int G>
const void* pick_staged(bool nt, bool mma) {
  if (mma)
    return nt ? reinterpret_cast<const void*>(&short_rows_staged_kernel<S, G, true, true>)
              : reinterpret_cast<const void*>(&short_rows_staged_kernel<S, G, false, true>);
  return nt ? reinterpret_cast<const void*>(&short_rows_staged_kernel<S, G, true, false>)
            : reinterpret_cast<const void*>(&short_rows_staged_kernel<S, G, false, false>);
}

// rows of at most 32 values: the direct kernel (8 groups per step); wider
// rows: the staged kernel with 4 or 8 groups per step
const void* short_rows_kernel_for(int s, int g, bool nt, bool mma) {
  if (s < kShortStagedMinLog2) {
    if (g != 8) return nullptr;
    switch (s) {
      case 0: return pick_direct<0>(nt, mma);
      case 1: return pick_direct<1>(nt, mma);
      case 2: return pick_direct<2>(nt, mma);
      default: return nullptr;
    }
  }
  if (g == 4) {
    switch (s) {
      case 3: return pick_staged<3, 4>(nt, mma);
      case 4: return pick_staged<4, 4>(nt, mma);
      case 5: return pick_staged<5, 4>(nt, mma);
      case 6: return pick_staged<6, 4>(nt, mma);
      default: return nullptr;
    }
  }
  if (g == 8) {
    switch (s) {
      case 3: return pick_staged<3, 8>(nt, mma);
      case 4: return pick_staged<4, 8>(nt, mma);
      case 5: return pick_staged<5, 8>(nt, mma);
      case 6: return pick_staged<6, 8>(nt, mma);
      default: return nullptr;
    }
  }
  return nullptr;
}

}  // namespace

hipError_t launch_short_rows(const Plan& plan, const void* x, float* out, hipStream_t stream) {
  if (plan.rows == 0) return hipSuccess;
  if (plan.n == 0 || plan.n > kChunk) return hipErrorInvalidValue;
  if ((plan.flags & ARMX_FLAG_MMA_LEAVES) && plan.waves * 64 > kShortMmaMaxBlock)
    return hipErrorInvalidValue;
  const void* fn = short_rows_kernel_for(plan.seg_log2, plan.r,
                                         (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0,
                                         (plan.flags & ARMX_FLAG_MMA_LEAVES) != 0);
  if (!fn) return hipErrorInvalidValue;
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  uint64_t rows = plan.rows, cols = plan.n, ld = plan.ld, chunk_rows = plan.chunk_rows;
  if (plan.seg_log2 >= kShortStagedMinLog2
          ? chunk_rows == 0 || chunk_rows > kShortChunkRows ||
                plan.lds_bytes < size_t(chunk_rows) * sizeof(float)
          : chunk_rows != 0)
    return hipErrorInvalidValue;
  if (plan.seg_log2 < kShortStagedMinLog2) {
    int remap = plan.xcd_remap;
    void* args[] = {&xh, &rows, &cols, &ld, &out, &remap};
    return launch_main(plan, fn, args, stream);
  }
  void* args[] = {&xh, &rows, &cols, &ld, &out, &chunk_rows};
  return launch_main(plan, fn, args, stream);
}

}  // namespace armx
