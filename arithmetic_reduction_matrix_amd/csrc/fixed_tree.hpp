// Building blocks of the fixed balanced-tree order, shared by the flat and the
// row-segmented fixed-order kernels.
//
// The tree ("Taming Bitwise Behavior in GPU Kernels with Tensor Core", arXiv
// 2609.11356, Abstract: a balanced-tree order makes a reduction reproducible;
// "GPU Tensor Cores for fast Arithmetic Reductions", arXiv 2001.05585,
// Abstract: 32-bit partials): leaves are the binary16 inputs widened exactly
// to binary32, padded with -0.0 to a power of two (the exact identity of
// round-to-nearest-even addition), and every node is one binary32 RNE
// addition of its two children.  A 512-value chunk (one wavefront load) is a
// complete depth-9 subtree; lane l holds leaves [8l, 8l + 8).
#pragma once

#include "device_common.hpp"
#include "plan.h"

namespace armx {
namespace dev {
namespace tree {

constexpr int kStack = kFixedMaxLog2Chunks + 1;

constexpr bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Level 1 of the tree for the two binary16 values in one 32-bit word:
// fl32(lo + hi).  v_fma_mix_f32 takes both halves as f16 operands (op_sel)
// and computes lo * 1.0 + hi with one round-to-nearest-even rounding; the
// product by 1.0 is exact, so the result is exactly the binary32 sum.  One
// instruction instead of two conversions and an add.
__device__ __forceinline__ float pair_node(uint32_t w) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(w));
  return r;
}

// Levels 1-7 of one chunk: this lane's 8 values (levels 1-3 in-lane), then
// lanes ^ 1, ^ 2 and the mirrors within 8 and 16 lanes (levels 4-7).  Every
// lane of a 16-lane row ends with that row's 128-value node.
__device__ __forceinline__ float chunk_rows(u32x4 t) {
  const float b0 = pair_node(t[0]) + pair_node(t[1]);
  const float b1 = pair_node(t[2]) + pair_node(t[3]);
  return lane_tree(b0 + b1, 4);
}

// Node of one chunk, from this lane's 8 values; identical in every lane.
__device__ __forceinline__ float chunk_node(u32x4 t) {
  return add_xor32(add_xor16(chunk_rows(t)));
}

// Node of one chunk in the order with MFMA leaves: one
// v_mfma_f32_16x16x32_f16 of the chunk against all-ones from a zero
// accumulator gives the 16 column sums (lane l holds column l % 16, and the
// four 16-lane rows hold the same values), then the balanced tree over the 16
// columns in column order (levels xor 1, xor 2, the mirror in 8 and the
// mirror in 16), so every lane ends with the chunk node.
__device__ __forceinline__ float chunk_node_mma(u32x4 t) {
  const floatx4 cols = mfma_ones(floatx4{0.0f, 0.0f, 0.0f, 0.0f}, t);
  return lane_tree(cols[0], 4);
}

// Node of a power-of-two group of R consecutive chunks in the order with
// MFMA leaves: the chunk nodes added pairwise in index order.
template <int R>
__device__ __forceinline__ float group_node_mma(const u32x4 (&v)[R]) {
  static_assert(is_pow2(R), "a group subtree needs a power-of-two R");
  float node[R];
#pragma unroll
  for (int r = 0; r < R; ++r) node[r] = chunk_node_mma(v[r]);
#pragma unroll
  for (int s = 1; s < R; s *= 2) {
#pragma unroll
    for (int i = 0; i < R; i += 2 * s) node[i] = node[i] + node[i + s];
  }
  return node[0];
}

// Node of a power-of-two group of R consecutive chunks (an aligned subtree of
// 512 R values), identical in every lane.  After levels 1-7 each chunk is four
// row nodes [c0 c1 c2 c3]; the remaining levels pair rows, halves and then
// chunks, two registers at a time, with the row and half permutes:
//   level 8  pair_rows16(A, B)     -> [A01 B01 A23 B23]
//   level 9  pair_halves32(AB, CD) -> [A B C D] (chunk nodes, one per row)
//   level 10 pair_rows16(ABCD, EFGH) -> [A+B E+F C+D G+H]
//   ... and so on, each add one node of the balanced tree.
template <int R>
__device__ __forceinline__ float group_node(const u32x4 (&v)[R]) {
  static_assert(R == 2 || R == 4 || R == 8, "packed group tree for R = 2, 4, 8");
  float rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = chunk_rows(v[r]);
  if constexpr (R == 2) {
    const float p = pair_rows16(rows[0], rows[1]);  // [A01 B01 A23 B23]
    const float q = add_xor32(p);                   // [A B A B]
    return add_xor16(q);                            // A+B everywhere
  } else if constexpr (R == 4) {
    const float p = pair_rows16(rows[0], rows[1]);  // [A01 B01 A23 B23]
    const float q = pair_rows16(rows[2], rows[3]);  // [C01 D01 C23 D23]
    const float c = pair_halves32(p, q);            // [A B C D]
    return add_xor32(add_xor16(c));                 // [A+B . C+D .] -> A+B+C+D
  } else {
    const float p0 = pair_rows16(rows[0], rows[1]);
    const float p1 = pair_rows16(rows[2], rows[3]);
    const float p2 = pair_rows16(rows[4], rows[5]);
    const float p3 = pair_rows16(rows[6], rows[7]);
    const float c0 = pair_halves32(p0, p1);         // [A B C D]
    const float c1 = pair_halves32(p2, p3);         // [E F G H]
    const float d = pair_rows16(c0, c1);            // [A+B E+F C+D G+H]
    return add_xor16(add_xor32(d));                 // [AB+CD EF+GH ..] -> all eight
  }
}

// Binary counter over aligned subtrees.  Pushing item g at level L (a node
// of 2^L consecutive chunks, g counting such nodes) completes m = (trailing
// one bits of g) groups: it absorbs stack levels L .. L+m-1 (lower indices on
// the left) and becomes stack level L+m.  Every stack index is a
// compile-time constant, so the stack lives in registers; m is small on
// average, so the chain of comparisons is short.
template <int L, int M>
__device__ __forceinline__ void merge_store(float (&stk)[kStack], float v) {
#pragma unroll
  for (int j = L; j < L + M; ++j) v = stk[j] + v;
  stk[L + M] = v;
}

template <int L, int M = 0>
__device__ __forceinline__ void push_switch(float (&stk)[kStack], int m, float v) {
  if constexpr (L + M >= kStack - 1) {
    merge_store<L, kStack - 1 - L>(stk, v);
  } else {
    if (m == M) {
      merge_store<L, M>(stk, v);
    } else {
      push_switch<L, M + 1>(stk, m, v);
    }
  }
}

template <int L>
__device__ __forceinline__ void counter_push_at(float (&stk)[kStack], uint64_t g, float v) {
  push_switch<L>(stk, __builtin_ctzll(~g), v);
}

__device__ __forceinline__ void counter_push(float (&stk)[kStack], uint64_t k, float v) {
  counter_push_at<0>(stk, k, v);
}

// Root of the tree over `count` pushed items padded with -0.0 subtrees:
// the stacked nodes of the set bits of count, joined from the smallest up.
__device__ __forceinline__ float counter_fold(const float (&stk)[kStack], uint64_t count) {
  float acc = -0.0f;
#pragma unroll
  for (int j = 0; j < kStack; ++j) {
    if ((count >> j) & 1) acc = stk[j] + acc;
  }
  return acc;
}

// Balanced tree over `count` values (padded with -0.0 to a power of two) with
// one block of T threads, T a power of two; result valid in thread 0.  The
// caller passes T as read at the start of its kernel: read here, after a
// completion ticket's atomics and fences, the block size is fetched from
// memory again (a round trip on the last block's path).
__device__ inline float tree_of_values(const float* vals, unsigned count, float* red,
                                       unsigned T) {
  unsigned p2 = 1;
  while (p2 < count) p2 <<= 1;
  const unsigned used = p2 < T ? p2 : T;   // threads with leaves
  const unsigned per = p2 / used;          // consecutive leaves per thread
  const unsigned t = threadIdx.x;
  float v = -0.0f;
  if (t < used) {
    float stk[kStack];
#pragma unroll
    for (int j = 0; j < kStack; ++j) stk[j] = -0.0f;
    // the leaves are pushed in order; their loads go out four at a time
    for (unsigned k0 = 0; k0 < per; k0 += 4) {
      float leaf[4];
#pragma unroll
      for (unsigned j = 0; j < 4; ++j) {
        const unsigned i = t * per + k0 + j;
        leaf[j] = (k0 + j < per && i < count) ? load_published(vals + i) : -0.0f;
      }
#pragma unroll
      for (unsigned j = 0; j < 4; ++j)
        if (k0 + j < per) counter_push(stk, k0 + j, leaf[j]);
    }
    v = counter_fold(stk, per);
  }
  int lv = 0;
  while ((1u << lv) < used && lv < 6) ++lv;
  v = lane_tree(v, lv);
  if (used <= 64) return v;
  // more than one wavefront: their nodes are consecutive; combine over lanes
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  const unsigned wu = used / 64;
  float w = -0.0f;
  if (wave_id() == 0) {
    w = unsigned(lane_id()) < wu ? red[lane_id()] : -0.0f;
    int l2 = 0;
    while ((1u << l2) < wu) ++l2;
    w = lane_tree(w, l2);
  }
  return w;
}

// Loads the R full chunks c0 .. c0 + R - 1.
template <int R, bool NT>
__device__ __forceinline__ void load_group(const u32x4* __restrict__ x, uint64_t c0, int lane,
                                           u32x4 (&v)[R]) {
  const u32x4* p = x + c0 * 64 + lane;
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = load16<NT>(p + r * 64);
}

// Nodes recorded per group of R chunks: one (the group's subtree root) when R
// is a power of two -- then a group of R consecutive, R-aligned chunks is a
// complete subtree -- else one per chunk.
template <int R>
constexpr int kNodesPerGroup = is_pow2(R) ? 1 : R;

// A wavefront's record of node values in index order, kept branch-free: the
// value (identical in every lane) is selected into lane (count % 64) of a
// slot register, and the slot register is stored as row count / 64 of this
// wavefront's LDS array on every record (one conflict-free ds_write).  A new
// row starts from -0.0, so a partly filled last row is already padded.
struct NodeLog {
  float* rows;        // this wavefront's LDS array
  float slots;        // current row, one node per lane
  unsigned count;     // nodes recorded

  __device__ __forceinline__ void record(float v, int lane) {
    const unsigned s = count & 63u;
    slots = unsigned(lane) == s ? v : (s == 0 ? -0.0f : slots);
    rows[(count & ~63u) + unsigned(lane)] = slots;
    ++count;
  }
};

// Reduces R loaded chunks (items k0 .. k0 + R - 1, k0 a multiple of R) and
// records their node(s): the group's subtree root for R = 2, 4, 8, else one
// node per chunk.  Straight-line code; nothing here branches.
// With MMA (the order with MFMA leaves) the chunk nodes come from
// chunk_node_mma and a power-of-two group adds them pairwise in index order.
template <int R, bool MMA = false>
__device__ __forceinline__ void reduce_group(const u32x4 (&v)[R], NodeLog& log, int lane) {
  if constexpr (MMA) {
    if constexpr (is_pow2(R)) {
      log.record(group_node_mma<R>(v), lane);
    } else {
      float node[R];
#pragma unroll
      for (int r = 0; r < R; ++r) node[r] = chunk_node_mma(v[r]);
#pragma unroll
      for (int r = 0; r < R; ++r) log.record(node[r], lane);
    }
  } else if constexpr (R == 1) {
    log.record(chunk_node(v[0]), lane);
  } else if constexpr (is_pow2(R)) {
    log.record(group_node<R>(v), lane);
  } else {
    float node[R];
#pragma unroll
    for (int r = 0; r < R; ++r) node[r] = chunk_node(v[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) log.record(node[r], lane);
  }
}

// Root of the balanced tree over vals[0 .. count) padded with -0.0 to a power
// of two, by one wavefront (every lane returns it).  Rows of 64 are complete
// subtrees: each is reduced with lane_tree and its root written back in
// place (row r's root to vals[r], after row r has been read), until one row
// is left.
__device__ inline float wave_tree(float* vals, unsigned count, int lane) {
  if (count == 0) return -0.0f;
  while (count > 64) {
    const unsigned rows = (count + 63) / 64;
    for (unsigned r = 0; r < rows; ++r) {
      const unsigned i = r * 64 + unsigned(lane);
      const float v = lane_tree_full(i < count ? vals[i] : -0.0f);
      if (lane == 0) vals[r] = v;
    }
    count = rows;
  }
  int lv = 0;
  while ((1u << lv) < count) ++lv;
  return lane_tree(unsigned(lane) < count ? vals[lane] : -0.0f, lv);
}


// Root of the subtree over chunks first .. first + valid - 1 of the n-value
// array x (leaves past n read as -0.0), by one wavefront (every lane returns
// it); the range must be the valid prefix of an aligned power-of-two range.
// `log_rows` is this wavefront's LDS node log.
template <int R, bool NT, int PACE = 0, bool MMA = false>
__device__ __forceinline__ float wave_range_root(const u32x4* __restrict__ x, uint64_t n,
                                                 uint64_t first, uint64_t valid, int lane,
                                                 float* log_rows) {
  NodeLog log{log_rows, -0.0f, 0u};

  // Chunks of this range that lie entirely below n, in groups of R, with a
  // software pipeline (ping-pong buffers, every load unconditional, whole
  // pairs of groups per iteration, a prefetch past the last group re-reads
  // it).  The loop body has no branches: a branch there lets the compiler
  // hoist the second group's reduction above the next prefetch and wait for
  // every load.
  const uint64_t full = n / 512;
  const uint64_t valid_full = first >= full ? 0 : (full - first < valid ? full - first : valid);
  const uint64_t groups = valid_full / R;
  uint64_t g = 0;
  if (groups > 0) {
    u32x4 a[R], b[R];
    load_group<R, NT>(x, first, lane, a);
    for (; g + 1 < groups; g += 2) {
      load_group<R, NT>(x, first + (g + 1) * R, lane, b);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the reduction
      reduce_group<R, MMA>(a, log, lane);
      pace_pause<PACE>();
      load_group<R, NT>(x, first + (g + 2 < groups ? g + 2 : g + 1) * R, lane, a);
      __builtin_amdgcn_sched_barrier(0);
      reduce_group<R, MMA>(b, log, lane);
      pace_pause<PACE>();
    }
    if (g < groups) {
      reduce_group<R, MMA>(a, log, lane);
      ++g;
    }
  }
  // The rest of the range (fewer than R chunks, the last one possibly
  // straddling n): its leaves past n are -0.0.  For a power-of-two R these
  // chunks and -0.0 chunks up to R form one more group subtree.
  if (g * R < valid) {
    float node[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint64_t k = g * R + r;
      node[r] = -0.0f;
      if (k < valid) {
        const uint64_t gk = first + k;
        const u32x4 v = gk < full ? load16<NT>(x + gk * 64 + lane)
                                  : load8_masked(reinterpret_cast<const uint16_t*>(x),
                                                 gk * 512 + uint64_t(lane) * 8, n, 0x8000u);
        if constexpr (MMA) {
          node[r] = chunk_node_mma(v);
        } else {
          node[r] = chunk_node(v);
        }
      }
    }
    if constexpr (is_pow2(R)) {
#pragma unroll
      for (int s = 1; s < R; s *= 2) {
#pragma unroll
        for (int i = 0; i < R; i += 2 * s) node[i] = node[i] + node[i + s];
      }
      log.record(node[0], lane);
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (g * R + r < valid) log.record(node[r], lane);
      }
    }
  }
  return wave_tree(log.rows, log.count, lane);
}

}  // namespace tree
}  // namespace dev
}  // namespace armx
