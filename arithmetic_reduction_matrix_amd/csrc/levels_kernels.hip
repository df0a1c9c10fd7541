// Free-order sum in the recursive all-MMA form.
//
// "GPU Tensor Cores for fast Arithmetic Reductions" (arXiv 2001.05585),
// Abstract: n numbers are reduced by chains of m x m MMAs, and the running
// time model T(n) = 5 log_{m^2}(n) counts levels of a recursion in which each
// level shrinks the data by about m^2 using MMAs alone.  Here every level is
// one launch, and a chain's reduction uses no cross-lane move, no LDS and no
// atomic: only MFMAs against all-ones operands.
//
// Level 1 (binary16 input).  A chain is R chunks of 512 values.  Each chunk,
// one 16-byte load per lane, is the A operand (16 x 32; lane l holds row
// l % 16, columns 8 (l / 16) .. + 7) of v_mfma_f32_16x16x32_f16 with B = ones,
// and the R products accumulate: D[i][j] = the sum of row i of the R tiles,
// the same for every column j.  In the accumulator layout lane j + 16 g holds
// D[4 g + r][j] in register r, so register r over the 64 lanes is a 4 x 16
// matrix whose row k is row sum 4 k + r: exactly a B operand (4 x 16) of
// v_mfma_f32_16x16x4_f32.  Four such MMAs with A = ones(16 x 4), chained over
// r = 0..3, add all 16 row sums: ones * (X * ones).  Every lane then holds the
// chain's total and lane 0 stores it -- one fp32 per chain, the chain
// sub-result the Abstract keeps in 32 bits.
//
// Level k >= 2 (the fp32 values of the level below).  A tile is 256 values,
// 4 per lane in one 16-byte load; value t of every lane forms the A operand
// (16 x 4; lane l holds row l % 16, column l / 16) of a v_mfma_f32_16x16x4_f32
// against ones, so four MMAs add a tile into 16 row sums; R tiles chain, and
// the same four ones * (row sums) MMAs finish the chain.  Levels repeat until
// one value is left, which is stored to out.
//
// The chains are fixed by n and R alone, so the result does not depend on
// the block size or the grid, and repeated calls give the same bits.
#include "device_common.hpp"
#include "launch.h"

namespace armx {
namespace {

using namespace dev;

// ones(16 x 4) * rows, chained over the four accumulator registers: the sum
// of the 16 row sums a 16 x 16 MFMA accumulator holds (valid in every lane).
__device__ __forceinline__ float ones_times_rows(floatx4 rows) {
  floatx4 t = {0.0f, 0.0f, 0.0f, 0.0f};
  t = __builtin_amdgcn_mfma_f32_16x16x4f32(1.0f, rows[0], t, 0, 0, 0);
  t = __builtin_amdgcn_mfma_f32_16x16x4f32(1.0f, rows[1], t, 0, 0, 0);
  t = __builtin_amdgcn_mfma_f32_16x16x4f32(1.0f, rows[2], t, 0, 0, 0);
  t = __builtin_amdgcn_mfma_f32_16x16x4f32(1.0f, rows[3], t, 0, 0, 0);
  return t[0];
}

// Total of a level-1 chain: R binary16 tiles as A operands against ones.
template <int R>
__device__ __forceinline__ float chain_total_f16(const u32x4 (&v)[R]) {
  const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
  floatx4 rows = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < R; ++r)
    rows = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, v[r]), ones, rows,
                                                  0, 0, 0);
  return ones_times_rows(rows);
}

// Total of a level-k chain: R fp32 tiles, four A operands each, against ones.
template <int R>
__device__ __forceinline__ float chain_total_f32(const floatx4 (&v)[R]) {
  floatx4 rows = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      rows = __builtin_amdgcn_mfma_f32_16x16x4f32(v[r][t], 1.0f, rows, 0, 0, 0);
  }
  return ones_times_rows(rows);
}

// Level 1 over the full chains c0, c0 + stride, ... (`iters` > 0 of them):
// the software pipeline of the free-order kernel (next chain's loads issued
// before the current chain's MMAs, ping-pong buffers, clamped unconditional
// prefetch), with each chain total stored one half-step later, after the
// next loads are in flight.  The first store writes a placeholder to chain
// c0's slot; the same lane overwrites it with chain c0's value later.
template <int R, bool NT>
__device__ __forceinline__ void stream_level1(const u32x4* __restrict__ x, uint64_t c0,
                                              uint64_t iters, uint64_t stride, int lane,
                                              float* __restrict__ vals) {
  const uint64_t last = c0 + (iters - 1) * stride;
  u32x4 a[R], b[R];
  float pv = 0.0f;
  uint64_t pc = c0;
  load_chain<R, NT>(x, c0, lane, a);
  const uint64_t pairs = iters / 2;
  for (uint64_t p = 0; p < pairs; ++p) {
    const uint64_t j = 2 * p;
    load_chain<R, NT>(x, c0 + (j + 1) * stride, lane, b);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the MMAs
    if (lane == 0) vals[pc] = pv;
    pv = chain_total_f16<R>(a);
    pc = c0 + j * stride;
    load_chain<R, NT>(x, j + 2 < iters ? c0 + (j + 2) * stride : last, lane, a);
    __builtin_amdgcn_sched_barrier(0);
    if (lane == 0) vals[pc] = pv;
    pv = chain_total_f16<R>(b);
    pc = c0 + (j + 1) * stride;
  }
  if (iters & 1) {  // a holds the last chain
    if (lane == 0) vals[pc] = pv;
    pv = chain_total_f16<R>(a);
    pc = last;
  }
  if (lane == 0) vals[pc] = pv;
}

// vals[c] = total of chain c (R x 512 values of x; values past n count as
// +0.0), for every c < ceil(n / (512 R)).  Wavefront g of T takes chains g,
// g + T, ...
template <int R, bool NT>
__global__ __launch_bounds__(1024) void level1_kernel(const u32x4* __restrict__ x, uint64_t n,
                                                      uint64_t chains_full,
                                                      float* __restrict__ vals) {
  const int lane = lane_id();
  const uint64_t T = uint64_t(gridDim.x) * uint64_t(num_waves());
  const uint64_t c0 = uint64_t(blockIdx.x) * uint64_t(num_waves()) + uint64_t(wave_id());
  const uint64_t iters = c0 < chains_full ? (chains_full - 1 - c0) / T + 1 : 0;
  if (iters > 0) stream_level1<R, NT>(x, c0, iters, T, lane, vals);
  const uint64_t c = c0 + iters * T;
  if (c == chains_full && chains_full * R * kChunk < n) {
    const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
    u32x4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint64_t e = (c * R + r) * kChunk + uint64_t(lane) * 8;
      v[r] = e < n ? load8_masked(xh, e, n, 0u) : u32x4{0u, 0u, 0u, 0u};
    }
    const float t = chain_total_f16<R>(v);
    if (lane == 0) vals[c] = t;
  }
}

// dst[c] = total of src[c 256 R .. (c + 1) 256 R) (values past count are
// +0.0), one chain per wavefront.
template <int R>
__global__ __launch_bounds__(1024) void levelk_kernel(const float* __restrict__ src,
                                                      uint64_t count, float* __restrict__ dst) {
  const int lane = lane_id();
  const uint64_t per_chain = uint64_t(R) * 256;
  const uint64_t c = uint64_t(blockIdx.x) * uint64_t(num_waves()) + uint64_t(wave_id());
  const uint64_t first = c * per_chain;
  if (first >= count) return;
  floatx4 v[R];
  if (first + per_chain <= count) {
    const floatx4* p = reinterpret_cast<const floatx4*>(src + first) + lane;
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = p[r * 64];
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint64_t e = first + uint64_t(r) * 256 + uint64_t(lane) * 4 + t;
        v[r][t] = e < count ? src[e] : 0.0f;
      }
    }
  }
  const float total = chain_total_f32<R>(v);
  if (lane == 0) dst[c] = total;
}

template <int R>
const void* pick_level1(bool nt) {
  return nt ? reinterpret_cast<const void*>(&level1_kernel<R, true>)
            : reinterpret_cast<const void*>(&level1_kernel<R, false>);
}

const void* level1_for(int r, bool nt) {
  switch (r) {
    case 1: return pick_level1<1>(nt);
    case 2: return pick_level1<2>(nt);
    case 3: return pick_level1<3>(nt);
    case 4: return pick_level1<4>(nt);
    case 5: return pick_level1<5>(nt);
    case 6: return pick_level1<6>(nt);
    case 7: return pick_level1<7>(nt);
    case 8: return pick_level1<8>(nt);
    default: return nullptr;
  }
}

const void* levelk_for(int r) {
  switch (r) {
    case 1: return reinterpret_cast<const void*>(&levelk_kernel<1>);
    case 2: return reinterpret_cast<const void*>(&levelk_kernel<2>);
    case 3: return reinterpret_cast<const void*>(&levelk_kernel<3>);
    case 4: return reinterpret_cast<const void*>(&levelk_kernel<4>);
    case 5: return reinterpret_cast<const void*>(&levelk_kernel<5>);
    case 6: return reinterpret_cast<const void*>(&levelk_kernel<6>);
    case 7: return reinterpret_cast<const void*>(&levelk_kernel<7>);
    case 8: return reinterpret_cast<const void*>(&levelk_kernel<8>);
    default: return nullptr;
  }
}

}  // namespace

hipError_t launch_levels(const Plan& plan, const void* x, float* out, void* ws,
                         hipStream_t stream) {
  if (plan.n == 0) return launch_zero(out, 1, stream);
  const void* f1 = level1_for(plan.r, (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0);
  const void* fk = levelk_for(plan.r);
  if (!f1 || !fk) return hipErrorInvalidValue;
  const uint64_t R = uint64_t(plan.r), W = uint64_t(plan.waves);
  // ping-pong level buffers after the workspace's counter region
  float* buf[2] = {nullptr, nullptr};
  if (ws) {
    char* base = static_cast<char*>(ws) + kCounterBytes;
    buf[0] = reinterpret_cast<float*>(base);
    buf[1] = reinterpret_cast<float*>(base + plan.partials_bytes);
  }
  uint64_t count = level_count(plan.n, R, 1);
  const u32x4* xv = static_cast<const u32x4*>(x);
  uint64_t n = plan.n;
  uint64_t chains_full = n / (R * kChunk);
  float* dst = count == 1 ? out : buf[0];
  hipEvent_t start = static_cast<hipEvent_t>(plan.start_event);
  hipEvent_t stop = static_cast<hipEvent_t>(plan.stop_event);
  void* args1[] = {&xv, &n, &chains_full, &dst};
  hipError_t e = launch_kernel(f1, dim3(unsigned(plan.grid)), dim3(unsigned(W * 64)), args1, 0,
                               stream, start, count == 1 ? stop : nullptr);
  int which = 0;
  while (e == hipSuccess && count > 1) {
    const float* src = dst;
    uint64_t src_count = count;
    count = level_count(count, R, 2);
    which ^= 1;
    dst = count == 1 ? out : buf[which];
    const uint64_t blocks = (count + W - 1) / W;
    void* args[] = {&src, &src_count, &dst};
    e = launch_kernel(fk, dim3(unsigned(blocks)), dim3(unsigned(W * 64)), args, 0, stream,
                      nullptr, count == 1 ? stop : nullptr);
  }
  return e;
}

}  // namespace armx
