// Device helpers for the gfx950 reduction kernels.
//
// Data layout used by every kernel: the input is a contiguous array of
// binary16 values.  One wavefront load is 64 lanes x 16 bytes: lane l reads
// the 8 consecutive values [8l, 8l + 8) of a 512-value "chunk", so a load is
// fully coalesced (1 KiB contiguous) and is exactly one 32 x 16 B operand of
// v_mfma_f32_16x16x32_f16.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "armx.h"

namespace armx {
namespace dev {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLanes = 64;

__device__ __forceinline__ int lane_id() { return int(threadIdx.x) & 63; }
// wave-uniform by construction; readfirstlane lets the compiler keep it (and
// everything derived from it) in scalar registers
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
}
__device__ __forceinline__ int num_waves() { return int(blockDim.x) >> 6; }

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

// 8 binary16 values starting at element e of xh (e a multiple of 8, xh
// 16-byte aligned); elements at or beyond n are replaced by `fill` (a
// binary16 bit pattern).  A lane whose 8 values all lie below n makes one
// 16-byte load, a lane entirely past n loads nothing, and only the lane that
// straddles n reads its values one by one.
__device__ __forceinline__ u32x4 load8_masked(const uint16_t* __restrict__ xh, uint64_t e,
                                              uint64_t n, uint32_t fill) {
  if (e + 8 <= n) return *reinterpret_cast<const u32x4*>(xh + e);
  const uint32_t f2 = fill | (fill << 16);
  if (e >= n) return u32x4{f2, f2, f2, f2};
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (e + i < n) ? uint32_t(xh[e + i]) : fill;
  u32x4 v;
  v[0] = h[0] | (h[1] << 16);
  v[1] = h[2] | (h[3] << 16);
  v[2] = h[4] | (h[5] << 16);
  v[3] = h[6] | (h[7] << 16);
  return v;
}

// 8 binary16 values starting at element e of xh, as load8_masked, but with
// no branch: every element is read (from index min(e + i, n - 1), so n must
// be at least 1) and those at or past n are replaced by `fill`.  Eight 2-byte
// loads per lane; for one-off reads outside a pipelined loop.
__device__ __forceinline__ u32x4 load8_clamped(const uint16_t* __restrict__ xh, uint64_t e,
                                               uint64_t n, uint32_t fill) {
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool in = e + i < n;
    const uint32_t v = xh[in ? e + i : n - 1];
    h[i] = in ? v : fill;
  }
  u32x4 v;
  v[0] = h[0] | (h[1] << 16);
  v[1] = h[2] | (h[3] << 16);
  v[2] = h[4] | (h[5] << 16);
  v[3] = h[6] | (h[7] << 16);
  return v;
}

// Blocks are dispatched to the 8 XCDs of an MI355X round-robin (block b to
// XCD b % 8), and every XCD has its own L2 and address-translation caches.
// This logical block id gives each XCD a contiguous range of ids, so that
// work assigned by consecutive ids (neighbouring rows) stays on one XCD.
constexpr uint64_t kXcds = 8;
__device__ __forceinline__ uint64_t xcd_block_id() {
  const uint64_t G = gridDim.x, b = blockIdx.x;
  const uint64_t per = G / kXcds, rem = G % kXcds, x = b % kXcds;
  return x * per + (x < rem ? x : rem) + b / kXcds;
}

// ---- cross-lane moves -------------------------------------------------------

__device__ __forceinline__ int fbits(float v) { return __builtin_bit_cast(int, v); }
__device__ __forceinline__ float bitsf(int v) { return __builtin_bit_cast(float, v); }

// DPP controls (GCN/CDNA encoding)
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i of each 8 reads lane 7 - i
constexpr int kDppMirror = 0x140;     // lane i of each 16 reads lane 15 - i
constexpr int kDppRor8 = 0x128;       // row_ror:8
constexpr int kDppRor4 = 0x124;
constexpr int kDppRor2 = 0x122;
constexpr int kDppRor1 = 0x121;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return bitsf(__builtin_amdgcn_update_dpp(0, fbits(v), CTRL, 0xF, 0xF, false));
}

// v + (v of lane l ^ 16): v_permlane16_swap exchanges the odd 16-lane rows of
// its first operand with the even rows of its second; with both operands v,
// the two results hold rows (0,0,2,2) and (1,1,3,3), so their sum pairs every
// lane with lane ^ 16.
__device__ __forceinline__ float add_xor16(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  return bitsf(int(p[0])) + bitsf(int(p[1]));
}

// v + (v of lane l ^ 32), by the same argument with v_permlane32_swap.
__device__ __forceinline__ float add_xor32(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
  return bitsf(int(p[0])) + bitsf(int(p[1]));
}

// Row-pair sums of two different registers at once.  With 16-lane rows
// a = [a0 a1 a2 a3] and b = [b0 b1 b2 b3] (each row holding one value),
// v_permlane16_swap(a, b) exchanges a's odd rows with b's even rows, so the
// two results are [a0 b0 a2 b2] and [a1 b1 a3 b3] and their sum is
// [a0+a1, b0+b1, a2+a3, b2+b3].
__device__ __forceinline__ float pair_rows16(float a, float b) {
  auto p = __builtin_amdgcn_permlane16_swap(fbits(a), fbits(b), false, false);
  return bitsf(int(p[0])) + bitsf(int(p[1]));
}

// Half sums of two different registers at once: with a = [alo ahi] and
// b = [blo bhi] (32-lane halves), v_permlane32_swap(a, b) gives [alo blo]
// and [ahi bhi], whose sum is [alo+ahi, blo+bhi].
__device__ __forceinline__ float pair_halves32(float a, float b) {
  auto p = __builtin_amdgcn_permlane32_swap(fbits(a), fbits(b), false, false);
  return bitsf(int(p[0])) + bitsf(int(p[1]));
}

// ---- fixed pairing ladder ---------------------------------------------------
//
// Level j (1-based) adds the values of aligned lane groups of size 2^(j-1)
// pairwise, provided every lane of a group already holds that group's value:
//   level 1: lane ^ 1, level 2: lane ^ 2 (quad permutes),
//   level 3: mirror within 8 lanes (reaches the other group of 4),
//   level 4: mirror within 16 lanes (reaches the other group of 8),
//   level 5: lane ^ 16, level 6: lane ^ 32.
// Both partners compute a + b or b + a, which are the same binary32 value, so
// after level j every lane of a group of 2^j holds the same node of a
// balanced binary tree over the lanes.  `levels` must be wave-uniform.
__device__ __forceinline__ float lane_tree(float v, int levels) {
  if (levels >= 1) v = v + dpp<kDppXor1>(v);
  if (levels >= 2) v = v + dpp<kDppXor2>(v);
  if (levels >= 3) v = v + dpp<kDppHalfMirror>(v);
  if (levels >= 4) v = v + dpp<kDppMirror>(v);
  if (levels >= 5) v = add_xor16(v);
  if (levels >= 6) v = add_xor32(v);
  return v;
}

__device__ __forceinline__ float lane_tree_full(float v) {
  v = v + dpp<kDppXor1>(v);
  v = v + dpp<kDppXor2>(v);
  v = v + dpp<kDppHalfMirror>(v);
  v = v + dpp<kDppMirror>(v);
  v = add_xor16(v);
  return add_xor32(v);
}

// Sum of the 16 lanes of each 16-lane row, in every lane of the row (the
// order differs between lanes; callers read one fixed lane).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppRor8>(v);
  v += dpp<kDppRor4>(v);
  v += dpp<kDppRor2>(v);
  v += dpp<kDppRor1>(v);
  return v;
}

// Sum over all 64 lanes (every lane gets the same value).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v = add_xor16(v);
  return add_xor32(v);
}

// ---- binary16 -> binary32 ---------------------------------------------------

__device__ __forceinline__ float lo_f32(uint32_t w) {
  return float(__builtin_bit_cast(half2v, w)[0]);
}
__device__ __forceinline__ float hi_f32(uint32_t w) {
  return float(__builtin_bit_cast(half2v, w)[1]);
}

// ---- the MFMA tile step -------------------------------------------------------
//
// acc += ONES(16x32) * T(32x16), with T the 512 values of one wavefront load.
// Lane l supplies column l % 16 of T, so acc (in every lane l) becomes the
// running sum of column l % 16, i.e. of the values loaded by the lanes
// congruent to l mod 16.  Products by 1.0 are exact; accumulation is fp32.
__device__ __forceinline__ floatx4 mfma_ones(floatx4 acc, u32x4 tile) {
  const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, __builtin_bit_cast(half8, tile), acc, 0,
                                                0, 0);
}

// The signed ones operand: A = 16 x 32 with rows 0-7 all +1 and rows 8-15 all
// -1.  Lane l supplies row l % 16 of A, so lanes with l % 16 >= 8 hold -1.
// Output row i of D = C + A * T then accumulates +(column sum) for i < 8 and
// -(column sum) for i >= 8; lane l holds rows 4 (l / 16) .. 4 (l / 16) + 3,
// so lanes 0-31 accumulate the + sums and lanes 32-63 the - sums of the
// same 16 columns, each output element on its own.  Products by -1.0 are
// exact, so the - elements are the same accumulations of the negated values.
__device__ __forceinline__ half8 signed_ones_operand() {
  const _Float16 s = (lane_id() & 8) ? _Float16(-1) : _Float16(1);
  return half8{s, s, s, s, s, s, s, s};
}

__device__ __forceinline__ floatx4 mfma_signed(floatx4 acc, u32x4 tile, half8 a) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8, tile), acc, 0, 0,
                                                0);
}

// Sum of one 16-byte load's 8 values, converted and added in fp32 (the
// MFMA-free design).
__device__ __forceinline__ void plain_add8(float& a, float& b, u32x4 t) {
  a += lo_f32(t[0]);
  b += hi_f32(t[0]);
  a += lo_f32(t[1]);
  b += hi_f32(t[1]);
  a += lo_f32(t[2]);
  b += hi_f32(t[2]);
  a += lo_f32(t[3]);
  b += hi_f32(t[3]);
}

// ---- request pacing -----------------------------------------------------------
//
// Measured on MI355X: a long persistent stream reads HBM faster when each
// wavefront pauses for a moment after reducing a chain, before issuing the
// next chain's loads -- with slightly fewer requests outstanding at once the
// memory system loses less to contention.  The pause is s_sleep PACE (about
// 64 PACE clocks); it changes no arithmetic.  2^28 MFMA sum: 76.8 us without,
// 74.9 us at PACE 8; fixed order at 2^30: 339 us without, 296 us at PACE 2.
// Short streams lose by it (the ramp and the tail dominate), so callers pick
// PACE from a wavefront's chain count.
template <int PACE>
__device__ __forceinline__ void pace_pause() {
  if constexpr (PACE > 0) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_sleep(PACE);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- streaming chains of tiles ----------------------------------------------

// Loads chain c of R chunks: R x 16 bytes per lane from base + c * R chunks.
template <int R, bool NT>
__device__ __forceinline__ void load_chain(const u32x4* __restrict__ base, uint64_t c, int lane,
                                           u32x4 (&v)[R]) {
  const u32x4* p = base + c * (uint64_t(R) * 64) + lane;
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = load16<NT>(p + r * 64);
}

// Designs of the free-order chain step (the template parameter D):
//   kSigned  MFMA against the signed ones operand (the default): lanes 0-31
//            carry the + column sums, lanes 32-63 the - column sums, and the
//            wavefront total is half their difference.  The MFMA's
//            accumulation cuts low bits toward minus infinity in some steps
//            (measured on gfx950), which leans a + sum low and a - sum high
//            by the same amount in distribution, so the difference cancels
//            the lean; at no extra instruction per load.
//   kPlain   the MFMA-free design: per-lane binary16 -> binary32 and fp32 adds.
//   kOnes    MFMA against the all-ones operand, every lane a + column sum
//            (the literal form; its results lean low on data of wide range).
constexpr int kSigned = 0;
constexpr int kPlain = 1;
constexpr int kOnes = 2;

// The design a call's flags select.
inline int chain_design(unsigned flags) {
  if (flags & ARMX_FLAG_PLAIN) return kPlain;
  if (flags & ARMX_FLAG_ALL_ONES) return kOnes;
  return kSigned;
}

// One chain: R tile steps whose fp32 result starts from zero; the caller adds
// it (one round-to-nearest-even v_add_f32) into the running per-lane sum.
// Keeping each chain's sub-result separate is what holds the error down: a
// single accumulator carried across many MFMAs grows large, and the MFMA's
// own accumulation then loses low bits on every step.
//   MFMA designs: lane l's chain value is the sum of column l % 16 of the R
//   tiles (kSigned: negated in lanes 32-63; the same value in all four
//   accumulator registers).
//   MFMA-free design: lane l's chain value is the sum of its own 8 R values.
template <int R, int D>
__device__ __forceinline__ float chain_value(const u32x4 (&v)[R]) {
  if constexpr (D == kPlain) {
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) plain_add8(a, b, v[r]);
    return a + b;
  } else if constexpr (D == kOnes) {
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < R; ++r) acc = mfma_ones(acc, v[r]);
    return acc[0];
  } else {
    const half8 a = signed_ones_operand();
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < R; ++r) acc = mfma_signed(acc, v[r], a);
    return acc[0];
  }
}

template <int R, int D>
__device__ __forceinline__ void chain_step(const u32x4 (&v)[R], float& run) {
  run += chain_value<R, D>(v);
}

// Accumulates the full chains c0, c0 + stride, ..., (`iters` of them).
// Software pipeline, unrolled by two with ping-pong buffers: the next chain's
// R loads are issued before the current chain's R tile steps, so a wavefront
// keeps up to 2R loads in flight and no registers are copied.  Every load in
// the loop is unconditional -- a branch around a load makes the compiler wait
// for all loads where the paths join -- so a prefetch past the last chain
// re-reads that chain (still in L2) and its values are not used.  A chain's
// value is added into `run` one half-step later, after the next loads are
// issued, so the wait for the MFMA chain's result never delays a prefetch.
// PACE > 0 pauses after every chain (pace_pause).
template <int R, bool NT, int D, int PACE = 0>
__device__ __forceinline__ void stream_chains(const u32x4* __restrict__ base, uint64_t c0,
                                              uint64_t iters, uint64_t stride, int lane,
                                              float& run) {
  if (iters == 0) return;
  if (iters == 1) {
    // a single chain (the one-chain-per-wavefront grid): no prefetch, so the
    // chain is not loaded again while its first load is still in flight
    u32x4 v[R];
    load_chain<R, NT>(base, c0, lane, v);
    run += chain_value<R, D>(v);
    return;
  }
  const uint64_t last = c0 + (iters - 1) * stride;
  u32x4 a[R], b[R];
  float pending = 0.0f;
  load_chain<R, NT>(base, c0, lane, a);
  for (uint64_t j = 0; j < iters; j += 2) {
    load_chain<R, NT>(base, j + 1 < iters ? c0 + (j + 1) * stride : last, lane, b);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the tile steps
    run += pending;
    pending = chain_value<R, D>(a);
    pace_pause<PACE>();
    load_chain<R, NT>(base, j + 2 < iters ? c0 + (j + 2) * stride : last, lane, a);
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 < iters) {
      run += pending;
      pending = chain_value<R, D>(b);
    }
    pace_pause<PACE>();
  }
  run += pending;
}

// The partial chain c (elements [c R 512, end) of a segment of `len` values
// starting at xh); values past `len` count as +0.0.
template <int R, int D>
__device__ __forceinline__ void tail_chain(const uint16_t* __restrict__ xh, uint64_t c,
                                           uint64_t len, int lane, float& run) {
  u32x4 v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint64_t e = (c * R + r) * 512 + uint64_t(lane) * 8;
    v[r] = e < len ? load8_masked(xh, e, len, 0u) : u32x4{0u, 0u, 0u, 0u};
  }
  chain_step<R, D>(v, run);
}

// The wavefront total of the running per-lane sums (valid in every lane).
template <int D>
__device__ __forceinline__ float wave_total(float run) {
  if constexpr (D == kPlain) {
    return wave_sum(run);
  } else if constexpr (D == kOnes) {
    // lanes 0..15 hold the 16 column totals (lanes 16..63 repeat them)
    return row16_sum(run);
  } else {
    // every 16-lane row sums its 16 columns: rows 0-1 (lanes 0-31) hold P,
    // the + total, rows 2-3 hold N, the - total; the total is (P - N) / 2
    // (one rounding; the halving is exact)
    const float t = row16_sum(run);
    const float p = bitsf(__builtin_amdgcn_readlane(fbits(t), 0));
    const float m = bitsf(__builtin_amdgcn_readlane(fbits(t), 32));
    return (p - m) * 0.5f;
  }
}

// ---- block combine and completion ticket ------------------------------------

// Sum of one value per wavefront (taken from lane 0) over the block; the result
// is valid in thread 0.  `red` is LDS of at least 16 floats.
__device__ __forceinline__ float block_sum_lane0(float t, float* red) {
  __syncthreads();  // red may still be read by a previous call
  if (lane_id() == 0) red[wave_id()] = t;
  __syncthreads();
  float v = 0.0f;
  if (wave_id() == 0) {
    v = lane_id() < num_waves() ? red[lane_id()] : 0.0f;
    v = row16_sum(v);
  }
  return v;
}

// Completion ticket.  Thread 0 publishes this block's result with `publish`
// (agent-scope atomic stores, written through to the level that all XCDs
// share), waits until those stores are complete (s_waitcnt vmcnt(0)), then
// increments `counter`.  The block whose increment is the `arrivals`-th one
// sees every other participant's result through agent-scope atomic loads.
// No agent-scope release fence is used: on gfx950 that fence writes back the
// whole L2 of the XCD, and one per block costs more than the reduction
// itself.  The last block returns the counter to zero for the next call on
// the same workspace.  Called by every thread; returns true in the last block
// only.
template <class Publish>
__device__ __forceinline__ bool publish_with_ticket(Publish publish, unsigned* counter,
                                                    unsigned arrivals, int* flag) {
  if (threadIdx.x == 0) {
    publish();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const unsigned prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == arrivals - 1;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// The ticket for one fp32 block result stored in `slot`.
__device__ __forceinline__ bool publish_and_check_last(float* slot, float value,
                                                       unsigned* counter, unsigned arrivals,
                                                       int* flag) {
  return publish_with_ticket(
      [&] { __hip_atomic_store(slot, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); },
      counter, arrivals, flag);
}

// A block result written by publish_and_check_last (or by an earlier kernel).
__device__ __forceinline__ float load_published(const float* slot) {
  return __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The last block of a split row reduction (rows x S parts published by
// wavefronts of many blocks, parts[r S + j] for j < S): stages every part in
// LDS (`stage`, at least rows x S floats) with eight loads in flight per
// thread, then writes out[r] = the balanced tree over row r's S parts in
// index order, padded with -0.0 to P, the power of two at or above S.  For
// P <= 64 a group of P lanes takes a row (64 / P rows per wavefront at a
// time); above, a wavefront takes a row with k = P / 64 parts per lane (at
// most 8), added pairwise in registers first.  Called by every thread of a
// block of `nt` threads (the size as read at the start of the kernel: read
// after the ticket it costs a memory round trip).
__device__ inline void combine_split_rows(const float* parts, uint64_t rows, unsigned S,
                                          float* __restrict__ out, float* stage, unsigned nt) {
  const uint64_t items = rows * S;
  for (uint64_t base = threadIdx.x; base < items; base += 8 * nt) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t i = base + uint64_t(j) * nt;
      v[j] = i < items ? load_published(parts + i) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t i = base + uint64_t(j) * nt;
      if (i < items) stage[i] = v[j];
    }
  }
  __syncthreads();
  int lp = 0;
  while ((1u << lp) < S) ++lp;
  const int lane = lane_id();
  const uint64_t W = uint64_t(nt) / 64;
  if (lp <= 6) {
    const uint64_t P = uint64_t(1) << lp, per_wave = uint64_t(64) >> lp;
    for (uint64_t r0 = uint64_t(wave_id()) * per_wave; r0 < rows; r0 += W * per_wave) {
      const uint64_t r = r0 + uint64_t(lane) / P, j = uint64_t(lane) % P;
      float v = r < rows && j < S ? stage[r * S + j] : -0.0f;
      v = lane_tree(v, lp);
      if (j == 0 && r < rows) out[r] = v;
    }
  } else {
    const uint64_t k = uint64_t(1) << (lp - 6);
    for (uint64_t r = uint64_t(wave_id()); r < rows; r += W) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint64_t i = uint64_t(lane) * k + uint64_t(j);
        v[j] = uint64_t(j) < k && i < S ? stage[r * S + i] : -0.0f;
      }
      // registers past k hold -0.0 subtrees, which leave every node unchanged
#pragma unroll
      for (int st = 1; st < 8; st *= 2) {
#pragma unroll
        for (int j = 0; j < 8; j += 2 * st) v[j] = v[j] + v[j + st];
      }
      const float root = lane_tree_full(v[0]);
      if (lane == 0) out[r] = root;
    }
  }
}

// Two-level completion.  Blocks form groups of `group` consecutive blocks (a
// power of two, at most kTicketGroups groups); each group has its own counter
// and the groups a top counter, so that no counter sees many increments and
// the atomics of different groups proceed in parallel: each counter sits in
// its own 256-byte stretch of the workspace (kTicketStride words), since
// device atomics on counters that share one are served one at a time.  The
// last block of a group combines the group's block results (in index order)
// into a group result; the last group combines the group results into out[0].
// `combine(values, count, red)` runs on every thread of the block and returns
// the combined value in thread 0.  Workspace: counters[0] is the top counter,
// counters[(1 + g) kTicketStride] group g's; all start (and end) at zero.
constexpr unsigned kTicketGroups = 255;
constexpr unsigned kTicketStride = 64;

//
// With one group of at least kSplitCountMinBlocks blocks and `split_count`
// (short streams, so that every block arrives at about the same time), only
// the counting is split: each run of 16 blocks has a counter, the last of each run counts
// on the top counter, and the last of those combines all the block results
// at once.  Measured on MI355X (256 blocks, graph-timed): at 2^24 values the
// free-order sum 9.65-9.95 -> 8.67-8.79 us and the fixed order 10.93 ->
// 10.02 us, since 256 increments of one counter, arriving together, are
// served one after another; at 2^26 and 2^28 the streams end spread out and
// the extra round trip costs 0.3-0.5 us, so longer streams keep one counter,
// and so do grids of fewer blocks (2^20 values, 64 blocks: 4.20 -> 4.57 us).
// Streams of fewer than kSplitCountChains chains (or fixed-order groups) per
// wavefront split their counting, in runs of kSplitCountRun blocks.
constexpr uint64_t kSplitCountChains = 16;
constexpr unsigned kSplitCountRun = 16;
constexpr unsigned kSplitCountMinBlocks = 128;

template <class Combine>
__device__ __forceinline__ void finish_two_level(float value, unsigned* counters,
                                                 float* partials, float* group_partials,
                                                 unsigned group, float* out, float* red,
                                                 int* flag, Combine combine,
                                                 bool split_count = false) {
  const unsigned b = blockIdx.x, G = gridDim.x;
  const unsigned g = b / group, g0 = g * group;
  const unsigned in_group = G - g0 < group ? G - g0 : group;
  const unsigned groups = (G + group - 1) / group;
  if (split_count && groups == 1 && G >= kSplitCountMinBlocks) {
    const unsigned runs = (G + kSplitCountRun - 1) / kSplitCountRun, s = b / kSplitCountRun;
    const unsigned in_run = G - s * kSplitCountRun < kSplitCountRun ? G - s * kSplitCountRun
                                                                    : kSplitCountRun;
    if (!publish_and_check_last(partials + b, value, counters + (1 + s) * kTicketStride, in_run,
                                flag)) return;
    __syncthreads();   // every thread has read the flag
    if (!publish_with_ticket([] {}, counters, runs, flag)) return;
    const float v = combine(partials, G, red);
    if (threadIdx.x == 0) out[0] = v;
    return;
  }
  if (!publish_and_check_last(partials + b, value, counters + (1 + g) * kTicketStride,
                              in_group, flag)) return;
  const float gv = combine(partials + g0, in_group, red);
  if (groups == 1) {
    if (threadIdx.x == 0) out[0] = gv;
    return;
  }
  __syncthreads();
  if (!publish_and_check_last(group_partials + g, gv, counters, groups, flag)) return;
  const float v = combine(group_partials, groups, red);
  if (threadIdx.x == 0) out[0] = v;
}

}  // namespace dev
}  // namespace armx
