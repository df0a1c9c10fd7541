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
//    -0.0) in the last block to finish, or by a second launch.
// The chain length R only sets how many chunk loads a wavefront has in
// flight; it never changes which values are added together.
#include "device_common.hpp"
#include "launch.h"

namespace armx {
namespace {

using namespace dev;

constexpr int kStack = kFixedMaxLog2Chunks + 1;

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

// Node of one chunk, from this lane's 8 values; identical in every lane.
__device__ __forceinline__ float chunk_node(u32x4 t) {
  const float b0 = pair_node(t[0]) + pair_node(t[1]);
  const float b1 = pair_node(t[2]) + pair_node(t[3]);
  return lane_tree_full(b0 + b1);
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
// one block whose size is a power of two; result valid in thread 0.
__device__ float tree_of_values(const float* vals, unsigned count, float* red) {
  unsigned p2 = 1;
  while (p2 < count) p2 <<= 1;
  const unsigned T = blockDim.x;
  const unsigned used = p2 < T ? p2 : T;   // threads with leaves
  const unsigned per = p2 / used;          // consecutive leaves per thread
  const unsigned t = threadIdx.x;
  float v = -0.0f;
  if (t < used) {
    float stk[kStack];
#pragma unroll
    for (int j = 0; j < kStack; ++j) stk[j] = -0.0f;
    for (unsigned k = 0; k < per; ++k) {
      const unsigned i = t * per + k;
      counter_push(stk, k, i < count ? load_published(vals + i) : -0.0f);
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

constexpr int log2_exact(int v) { return v <= 1 ? 0 : 1 + log2_exact(v / 2); }

// Reduces R loaded chunks, items k0 .. k0 + R - 1 of the range (k0 a multiple
// of R), and appends their nodes in index order.  The R chunk trees are
// independent and computed first, so their instructions interleave.  When R
// is a power of two the R nodes form an aligned subtree: it is finished in
// registers and pushed once at level log2(R).
template <int R>
__device__ __forceinline__ void reduce_group(const u32x4 (&v)[R], float (&stk)[kStack],
                                             uint64_t k0) {
  float node[R];
#pragma unroll
  for (int r = 0; r < R; ++r) node[r] = chunk_node(v[r]);
  if constexpr ((R & (R - 1)) == 0) {
#pragma unroll
    for (int s = 1; s < R; s *= 2) {
#pragma unroll
      for (int i = 0; i < R; i += 2 * s) node[i] = node[i] + node[i + s];
    }
    counter_push_at<log2_exact(R)>(stk, k0 / R, node[0]);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) counter_push(stk, k0 + r, node[r]);
  }
}

template <int R, bool NT>
__global__ __launch_bounds__(1024) void fixed_kernel(const u32x4* __restrict__ x, uint64_t n,
                                                     int log2c, float* __restrict__ roots,
                                                     unsigned* __restrict__ counter,
                                                     float* __restrict__ out, int two_pass) {
  __shared__ float red[16];
  __shared__ int flag;
  const int lane = lane_id();
  const int W = num_waves();
  const uint64_t chunks = (n + 511) / 512;
  const uint64_t first = (uint64_t(blockIdx.x) * W + uint64_t(wave_id())) << log2c;
  const uint64_t span = uint64_t(1) << log2c;
  const uint64_t valid = first >= chunks ? 0 : (chunks - first < span ? chunks - first : span);

  float stk[kStack];
#pragma unroll
  for (int j = 0; j < kStack; ++j) stk[j] = -0.0f;
  // Chunks of this range that lie entirely below n, processed in groups of
  // R with a software pipeline (ping-pong buffers; every load unconditional,
  // a prefetch past the last group re-reads that group); then the rest one
  // by one.
  const uint64_t full = n / 512;
  const uint64_t valid_full = first >= full ? 0 : (full - first < valid ? full - first : valid);
  const uint64_t groups = valid_full / R;
  if (groups > 0) {
    u32x4 a[R], b[R];
    load_group<R, NT>(x, first, lane, a);
    for (uint64_t g = 0; g < groups; g += 2) {
      load_group<R, NT>(x, first + (g + 1 < groups ? g + 1 : groups - 1) * R, lane, b);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the reduction
      reduce_group<R>(a, stk, g * R);
      load_group<R, NT>(x, first + (g + 2 < groups ? g + 2 : groups - 1) * R, lane, a);
      __builtin_amdgcn_sched_barrier(0);
      if (g + 1 < groups) reduce_group<R>(b, stk, (g + 1) * R);
    }
  }
  for (uint64_t k = groups * R; k < valid; ++k) {
    const uint64_t gk = first + k;
    const u32x4 v = gk < full ? load16<NT>(x + gk * 64 + lane)
                              : load8_masked(reinterpret_cast<const uint16_t*>(x),
                                             gk * 512 + uint64_t(lane) * 8, n, 0x8000u);
    counter_push(stk, k, chunk_node(v));
  }
  const float wave_root = counter_fold(stk, valid);

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
  if (!publish_and_check_last(roots + blockIdx.x, block_root, counter, &flag)) return;
  const float root = tree_of_values(roots, gridDim.x, red);
  if (threadIdx.x == 0) out[0] = root;
}

__global__ __launch_bounds__(1024) void fixed_final_kernel(const float* __restrict__ roots,
                                                           unsigned count,
                                                           float* __restrict__ out) {
  __shared__ float red[16];
  const float root = tree_of_values(roots, count, red);
  if (threadIdx.x == 0) out[0] = root;
}

template <int R>
const void* pick_fixed(bool nt) {
  return nt ? reinterpret_cast<const void*>(&fixed_kernel<R, true>)
            : reinterpret_cast<const void*>(&fixed_kernel<R, false>);
}

const void* fixed_kernel_for(int r, bool nt) {
  switch (r) {
    case 1: return pick_fixed<1>(nt);
    case 2: return pick_fixed<2>(nt);
    case 3: return pick_fixed<3>(nt);
    case 4: return pick_fixed<4>(nt);
    case 5: return pick_fixed<5>(nt);
    case 6: return pick_fixed<6>(nt);
    case 7: return pick_fixed<7>(nt);
    case 8: return pick_fixed<8>(nt);
    default: return nullptr;
  }
}

}  // namespace

hipError_t launch_fixed(const Plan& plan, const void* x, float* out, void* ws,
                        hipStream_t stream) {
  if (plan.n == 0) return launch_zero(out, 1, stream);
  const void* fn = fixed_kernel_for(plan.r, (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0);
  if (!fn) return hipErrorInvalidValue;
  const u32x4* xv = static_cast<const u32x4*>(x);
  uint64_t n = plan.n;
  int log2c = plan.log2_chunks;
  unsigned* counter = static_cast<unsigned*>(ws);
  float* roots = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  int two_pass = (plan.flags & ARMX_FLAG_TWO_PASS) ? 1 : 0;
  void* args[] = {&xv, &n, &log2c, &roots, &counter, &out, &two_pass};
  hipError_t e = hipLaunchKernel(fn, dim3(unsigned(plan.grid)), dim3(unsigned(plan.waves * 64)),
                                 args, 0, stream);
  if (e != hipSuccess || !two_pass || plan.grid == 1) return e;
  unsigned count = unsigned(plan.grid);
  const float* croots = roots;
  // the final tree needs a power-of-two block: 1024 threads
  void* fargs[] = {&croots, &count, &out};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fixed_final_kernel), dim3(1), dim3(1024),
                         fargs, 0, stream);
}

}  // namespace armx
