// Exact, order-free sum: out = the binary32 nearest (ties to even) to the
// real sum of x[0..n), and optionally that sum itself as a 128-bit integer
// count of 2^-24.
//
// Every finite binary16 value is an integer multiple of 2^-24 below 2^16 in
// magnitude, so the sum is an integer count of 2^-24 units, and integer
// addition is associative: every grouping of the additions gives the same
// total, whatever the block size, chain length, grid or device.  The
// kernel keeps every step exact:
//  * per lane and chain (R loads, 8 R values) the values are widened to
//    binary64 and added; every partial sum is a multiple of 2^-24 below
//    8 R 2^16 <= 2^22, which a 53-bit significand holds exactly;
//  * the chain total t = s 2^24 (an integer below 2^46) is split into two
//    limbs, t = h 2^32 + l with 0 <= l < 2^32, and each limb is added into
//    its own 64-bit integer accumulator -- numbers carried as narrow
//    components with fixed weights (1 and 2^32) and recombined exactly at the
//    end, the limb representation of "AWE: Adaptive Weight Encoding for Exact
//    Integer Matrix Products with Fewer GEMMs on FP4 Tensor Cores" (arXiv
//    2609.24519, Abstract) applied to a sum; neither accumulator can
//    overflow for n <= 2^40;
//  * wavefront, block and grid combines add these integers, folding the low
//    limb's carries into the high one so every term stays below 2^32; the
//    last block (completion ticket) rounds the 128-bit total once.
// That default form uses no MFMA.  ARMX_FLAG_INT_LIMBS selects the form
// whose sums are integer MFMAs over 8-bit limbs (the limb planes of the AWE
// Abstract): every value's count q (|q| < 2^40) is written as eight signed
// 8-bit digits d_0 .. d_7 (the bytes of its two's complement with their top
// bits flipped; see value_digits), and v_mfma_i32_16x16x64_i8 against a
// digit-selector operand adds, per output column, the digits of each
// position m over 8 values per MFMA -- exact in 32-bit integers -- so the
// digit planes are summed by the matrix cores and recombined at the end:
// positions 0-4 with their weights 2^(8m), plus a constant per value and a
// term per negative value, whose count position 7 gives.  Building the
// digits costs about 14 vector instructions per value, against three for
// the binary64 form.
//
// Non-finite inputs: a chain whose binary64 sum is not finite sets a flag
// (+Inf, -Inf or NaN) instead of adding to the integers; the result follows
// IEEE addition (NaN if any NaN or both infinities, else the infinity), and
// the 128-bit output is then 0.
#include <type_traits>

#include "device_common.hpp"
#include "launch.h"

namespace armx {
namespace {

using namespace dev;

constexpr unsigned kPosInf = 1, kNegInf = 2, kNaN = 4;

// A partial sum: hi 2^32 + lo units of 2^-24, plus the non-finite flags.
struct Exact {
  int64_t hi;
  uint64_t lo;
  unsigned flags;
};

// Moves the carries of lo into hi, leaving 0 <= lo < 2^32.
__device__ __forceinline__ void fold(Exact& a) {
  a.hi += int64_t(a.lo >> 32);
  a.lo &= 0xFFFFFFFFull;
}

template <int R>
__device__ __forceinline__ void add_chain(const u32x4 (&v)[R], Exact& a) {
  double s0 = 0.0, s1 = 0.0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s0 += double(lo_f32(v[r][w]));
      s1 += double(hi_f32(v[r][w]));
    }
  }
  const double s = s0 + s1;
  const bool finite = __builtin_isfinite(s);
  a.flags |= finite ? 0u : (s != s ? kNaN : (s > 0.0 ? kPosInf : kNegInf));
  const double t = finite ? s * 0x1p24 : 0.0;
  const double h = __builtin_floor(t * 0x1p-32);
  const double l = __builtin_fma(-h, 0x1p32, t);
  a.hi += int64_t(int(h));
  a.lo += uint64_t(unsigned(l));
}

// ---- the integer-MFMA limb form ------------------------------------------
//
// Digits of one value.  A finite binary16 value is q 2^-24 with q = +-M 2^t,
// M = the significand with its hidden bit (f, or 1024 + f), t = e - 1 (0 for
// subnormals, e the exponent field), |q| < 2^40.  Let g = |q| xor (all ones
// if negative): g = q for q >= 0 and g = q - 1 for q < 0, in two's
// complement.  The digits are the bytes g_m of g with their top bit flipped,
// read as signed 8-bit integers: d_m = g_m - 128 (in [-128, 127]).  Bytes
// 0-4 hold g mod 2^40 = q, or 2^40 + q - 1 for a negative value, so
//   q = sum_{m<5} d_m 2^(8m) + C40 + [q < 0] (1 - 2^40),
// C40 = 0x8080808080; bytes 5-7 are all 0x00 (d = -128) for q >= 0 and all
// 0xFF (d = 127) for q < 0, so the sum of digit 7 over N values is
// 255 #negative - 128 N, which counts the negative values.  The eight
// digits are returned as the bytes of one 64-bit word (digit m in byte m):
// the flip and the sign are one xor with (all ones if negative) xor
// 0x80...80.  An exponent field of 31 (infinity, NaN) gives digits of no
// meaning; such chains are flagged apart.
// Half HI (0 or 1) of the 32-bit word w holds the value; `e` receives its
// exponent field.
template <int HI>
__device__ __forceinline__ uint64_t value_digits(uint32_t w, uint32_t& e) {
  e = (w >> (10 + 16 * HI)) & 31u;
  const uint32_t f = (w >> (16 * HI)) & 1023u;
  const int32_t sign = HI ? int32_t(w) >> 31 : int32_t(w << 16) >> 31;   // 0 or -1
  const uint32_t mn = __builtin_elementwise_min(e, 1u);
  const uint32_t m = (mn << 10) | f;
  const uint64_t mag = uint64_t(m) << (e - mn);
  const uint32_t k = uint32_t(sign) ^ 0x80808080u;
  return mag ^ (uint64_t(k) << 32 | k);
}

typedef int int4v __attribute__((ext_vector_type(4)));

// The digit selector: A of v_mfma_i32_16x16x64_i8 with A[i][k] = 1 when
// k mod 8 == i < 8, else 0.  Lane l supplies row l % 16 over 16 K positions
// (two 8-aligned runs of K, byte b at a K index congruent to b mod 8), so
// its bytes b and b + 8 with b == l % 16 are 1 for l % 16 < 8; rows 8-15 are
// zero.  Output row i (< 8) of column j then adds digit i of the 8 values
// whose digits fill column j of B.
__device__ __forceinline__ int4v digit_selector(int lane) {
  const int i = lane & 15;
  int4v a = {0, 0, 0, 0};
  if (i < 8) {
    const int one = 1 << (8 * (i & 3));
    a[i >> 2] = one;
    a[(i >> 2) + 2] = one;
  }
  return a;
}

// Per-lane state of the limb form: the digit-position sums of this lane's
// accumulator rows (lane l holds rows 4 (l / 16) .. + 3 of column l % 16:
// digit positions 0-3 in lanes 0-15, 4-7 in lanes 16-31, zero in lanes
// 32-63), and the largest exponent field it loaded (31: an infinity or a
// NaN).
struct LimbSums {
  int64_t pos[4];
  uint32_t expo;   // the largest exponent field (0-31) of any value seen
};

// One chain of R loads (8 R values per lane): 4 R integer MFMAs (two values'
// digits, 16 bytes, per lane each) into two accumulators in turn (so that
// consecutive MFMAs do not wait for each other), exact in 32 bits within the
// chain (8 digits of at most 128 in magnitude per element per MFMA), then
// added into the 64-bit sums.  Every output column takes 8 values per MFMA,
// 32 per load.  Values with exponent field 31 (infinity, NaN) give digits
// of no meaning; the largest exponent field is kept, and a wavefront that
// saw 31 works out the non-finite flags after its stream.
template <int R>
__device__ __forceinline__ void add_chain_limbs(const u32x4 (&v)[R], const int4v sel,
                                                LimbSums& ls) {
  int4v acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  uint32_t expo = ls.expo;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int w = 0; w < 4; w += 2) {
      uint32_t e0, e1, e2, e3;
      const uint64_t d0 = value_digits<0>(v[r][w], e0);
      const uint64_t d1 = value_digits<1>(v[r][w], e1);
      const uint64_t d2 = value_digits<0>(v[r][w + 1], e2);
      const uint64_t d3 = value_digits<1>(v[r][w + 1], e3);
      const int4v b01 = {int(uint32_t(d0)), int(uint32_t(d0 >> 32)), int(uint32_t(d1)),
                         int(uint32_t(d1 >> 32))};
      const int4v b23 = {int(uint32_t(d2)), int(uint32_t(d2 >> 32)), int(uint32_t(d3)),
                         int(uint32_t(d3 >> 32))};
      acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(sel, b01, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(sel, b23, acc1, 0, 0, 0);
      expo = __builtin_elementwise_max(expo, __builtin_elementwise_max(e0, e1));
      expo = __builtin_elementwise_max(expo, __builtin_elementwise_max(e2, e3));
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) ls.pos[r] += int64_t(acc0[r]) + int64_t(acc1[r]);
  ls.expo = expo;
}

// The lane's limb sums as an Exact, after `loads` loads per lane (N = 32
// loads values per output column): positions 0-4 weigh 2^(8m); the lane of
// positions 4-7 of a column adds N C40 and, with the column's negative
// count #neg = (D7 + 128 N) / 255 from its digit-7 sum D7, #neg (1 - 2^40).
__device__ __forceinline__ void limbs_to_exact(const LimbSums& ls, int lane, uint64_t loads,
                                               Exact& a) {
  if ((lane >> 4) & 2) return;   // lanes 32-63 hold zeros
  if (((lane >> 4) & 1) == 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t t = int64_t(uint64_t(ls.pos[m]) << (8 * m));
      a.hi += t >> 32;
      a.lo += uint64_t(t) & 0xFFFFFFFFull;
    }
  } else {
    const uint64_t N = 32 * loads;
    const uint64_t neg = uint64_t(ls.pos[3] + int64_t(128 * N)) / 255u;
    a.hi += ls.pos[0];                                   // digit 4: 2^32
    a.hi += int64_t(N * 0x80u) - int64_t(neg << 8);      // N C40 and -#neg 2^40
    a.lo += N * 0x80808080ull + neg;
  }
}

// The full chains c0, c0 + stride, ... (`iters` of them), with the load
// pipeline of the free-order kernel: the next chain's loads are issued before
// the current chain's additions, ping-pong buffers, clamped prefetch.
template <int R, bool NT, bool LIMBS>
__device__ __forceinline__ void stream_exact(const u32x4* __restrict__ x, uint64_t c0,
                                             uint64_t iters, uint64_t stride, int lane,
                                             Exact& a, LimbSums& ls) {
  if (iters == 0) return;
  const int4v sel = digit_selector(lane);
  auto add = [&](const u32x4 (&v)[R]) {
    if constexpr (LIMBS) {
      add_chain_limbs<R>(v, sel, ls);
    } else {
      add_chain<R>(v, a);
    }
  };
  const uint64_t last = c0 + (iters - 1) * stride;
  u32x4 p[R], q[R];
  load_chain<R, NT>(x, c0, lane, p);
  const uint64_t pairs = iters / 2;
  for (uint64_t k = 0; k < pairs; ++k) {
    const uint64_t j = 2 * k;
    load_chain<R, NT>(x, c0 + (j + 1) * stride, lane, q);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the additions
    add(p);
    load_chain<R, NT>(x, j + 2 < iters ? c0 + (j + 2) * stride : last, lane, p);
    __builtin_amdgcn_sched_barrier(0);
    add(q);
  }
  if (iters & 1) add(p);  // p holds the last chain
}

// One 32-bit word of lane (lane within its row rotated right by CTRL's amount).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_word(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return uint64_t(dpp_word<CTRL>(uint32_t(v >> 32))) << 32 | dpp_word<CTRL>(uint32_t(v));
}

// a + (a of another lane), the other lane's words given as they arrived.
__device__ __forceinline__ void add_words(Exact& a, uint32_t hh, uint32_t hl, uint32_t lh,
                                          uint32_t ll, uint32_t f) {
  a.hi += int64_t(uint64_t(hh) << 32 | hl);
  a.lo += uint64_t(lh) << 32 | ll;
  a.flags |= f;
}

// The two halves of a lane-pair exchange (v_permlane16_swap or
// v_permlane32_swap with both operands the same register): p[0] + p[1] pairs
// every lane with lane ^ 16 (or ^ 32) for any commutative operation.
template <bool X32>
__device__ __forceinline__ Exact add_swapped(const Exact& a) {
  auto sw = [](uint32_t v) {
    if constexpr (X32) {
      return __builtin_amdgcn_permlane32_swap(v, v, false, false);
    } else {
      return __builtin_amdgcn_permlane16_swap(v, v, false, false);
    }
  };
  const auto hh = sw(uint32_t(uint64_t(a.hi) >> 32)), hl = sw(uint32_t(uint64_t(a.hi)));
  const auto lh = sw(uint32_t(a.lo >> 32)), ll = sw(uint32_t(a.lo));
  const auto f = sw(a.flags);
  Exact r{int64_t(uint64_t(hh[0]) << 32 | hl[0]), uint64_t(lh[0]) << 32 | ll[0], f[0]};
  add_words(r, hh[1], hl[1], lh[1], ll[1], f[1]);
  return r;
}

// Sum over the 64 lanes (every lane gets it); any order, the sums are exact.
// Row rotations (DPP) within each 16-lane row, then the row pairs and halves
// exchanged with the permlane swaps: no LDS round trips.
__device__ __forceinline__ Exact wave_exact(Exact a) {
  auto rot = [&](auto ctl) {
    constexpr int C = decltype(ctl)::value;
    const uint64_t h = dpp_u64<C>(uint64_t(a.hi)), l = dpp_u64<C>(a.lo);
    const uint32_t f = dpp_word<C>(a.flags);
    a.hi += int64_t(h);
    a.lo += l;
    a.flags |= f;
  };
  rot(std::integral_constant<int, kDppRor8>{});
  rot(std::integral_constant<int, kDppRor4>{});
  rot(std::integral_constant<int, kDppRor2>{});
  rot(std::integral_constant<int, kDppRor1>{});
  a = add_swapped<false>(a);
  a = add_swapped<true>(a);
  fold(a);
  return a;
}

// Sum over the block's wavefronts (lane 0's values); valid in wavefront 0.
struct ExactLds {
  int64_t hi[16];
  uint64_t lo[16];
  unsigned flags[16];
};

__device__ __forceinline__ Exact block_exact(Exact a, ExactLds& s) {
  __syncthreads();  // s may still be read by a previous call
  if (lane_id() == 0) {
    s.hi[wave_id()] = a.hi;
    s.lo[wave_id()] = a.lo;
    s.flags[wave_id()] = a.flags;
  }
  __syncthreads();
  Exact r{0, 0, 0};
  if (wave_id() == 0) {
    if (lane_id() < num_waves()) r = Exact{s.hi[lane_id()], s.lo[lane_id()], s.flags[lane_id()]};
    r = wave_exact(r);
  }
  return r;
}

// A published partial: 4 x 64-bit words (hi, lo, flags, unused).
constexpr int kRecordWords = 4;

__device__ __forceinline__ void store_record(uint64_t* rec, const Exact& a) {
  __hip_atomic_store(rec + 0, uint64_t(a.hi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(rec + 1, a.lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(rec + 2, uint64_t(a.flags), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of `count` published records; valid in wavefront 0.
// (records loaded two per thread at a time, so that their loads are in
// flight together; the sums are exact, so the order does not matter)
__device__ Exact combine_records(const uint64_t* recs, unsigned count, ExactLds& s) {
  Exact a{0, 0, 0};
  const unsigned B = blockDim.x;
  for (unsigned i0 = threadIdx.x; i0 < count; i0 += 2 * B) {
    uint64_t w[2][3];
#pragma unroll
    for (unsigned k = 0; k < 2; ++k) {
      const unsigned i = i0 + k * B;
      const uint64_t* r = recs + uint64_t(i) * kRecordWords;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        w[k][j] = i < count ? __hip_atomic_load(r + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0;
    }
#pragma unroll
    for (unsigned k = 0; k < 2; ++k) {
      a.hi += int64_t(w[k][0]);
      a.lo += w[k][1];
      a.flags |= unsigned(w[k][2]);
    }
  }
  fold(a);
  return block_exact(wave_exact(a), s);
}

// The binary32 nearest to (hi 2^64 + lo) 2^-24 (a 128-bit two's complement
// count), ties to even; +0.0 for zero.  |value| < 2^57 here, so the result is
// finite and normal or zero.
__device__ float round_to_binary32(int64_t hi, uint64_t lo) {
  const bool neg = hi < 0;
  unsigned __int128 m = (unsigned __int128)(uint64_t(hi)) << 64 | lo;
  if (neg) m = ~m + 1;
  if (m == 0) return 0.0f;
  const uint64_t mh = uint64_t(m >> 64), ml = uint64_t(m);
  const int p = mh ? 127 - __builtin_clzll(mh) : 63 - __builtin_clzll(ml);  // top bit
  uint32_t keep;
  int e;
  if (p < 24) {
    keep = uint32_t(ml);
    e = -24;
  } else {
    const int shift = p - 23;
    keep = uint32_t(m >> shift);
    const unsigned __int128 rem = m & ((((unsigned __int128)1) << shift) - 1);
    const unsigned __int128 half = ((unsigned __int128)1) << (shift - 1);
    if (rem > half || (rem == half && (keep & 1u))) ++keep;
    e = shift - 24;
    if (keep == (1u << 24)) {
      keep >>= 1;
      ++e;
    }
  }
  const float r = __builtin_ldexpf(float(keep), e);
  return neg ? -r : r;
}

__device__ void finish_exact(Exact a, float* out, int64_t* out_fixed) {
  fold(a);
  const uint64_t t_lo = (uint64_t(a.hi) << 32) | a.lo;
  const int64_t t_hi = a.hi >> 32;
  float r;
  if ((a.flags & kNaN) || ((a.flags & kPosInf) && (a.flags & kNegInf))) {
    r = __builtin_nanf("");
  } else if (a.flags & kPosInf) {
    r = __builtin_inff();
  } else if (a.flags & kNegInf) {
    r = -__builtin_inff();
  } else {
    r = round_to_binary32(t_hi, t_lo);
  }
  out[0] = r;
  if (out_fixed) {
    out_fixed[0] = a.flags ? 0 : int64_t(t_lo);
    out_fixed[1] = a.flags ? 0 : t_hi;
  }
}

// The limb form needs more than the 128 registers per lane a 1024-thread
// block leaves (its chain holds 16 R digit words besides the loads), so its
// blocks are bounded to kExactLimbsMaxBlock threads (the plan lowers larger
// requests; the result never depends on the block size).
template <int R, bool NT, bool LIMBS>
__global__ __launch_bounds__(LIMBS ? kExactLimbsMaxBlock : 1024) void exact_kernel(const u32x4* __restrict__ x, uint64_t n,
                                                     uint64_t chains_full,
                                                     unsigned* __restrict__ counters,
                                                     uint64_t* __restrict__ partials,
                                                     uint64_t* __restrict__ group_partials,
                                                     unsigned group, float* __restrict__ out,
                                                     int64_t* __restrict__ out_fixed) {
  __shared__ ExactLds lds;
  __shared__ int flag;
  const int lane = lane_id();
  const uint64_t W = uint64_t(num_waves());
  const uint64_t total_waves = uint64_t(gridDim.x) * W;
  uint64_t c = uint64_t(blockIdx.x) * W + uint64_t(wave_id());

  Exact a{0, 0, 0};
  LimbSums ls{{0, 0, 0, 0}, 0};
  const uint64_t c0 = c;
  const uint64_t iters = c < chains_full ? (chains_full - 1 - c) / total_waves + 1 : 0;
  // No request pacing (pace_pause): the binary64 additions already space a
  // wavefront's requests, and a pause on top lost (2^28: 76.0 -> 88.7 us at
  // the free-order sum's pauses).
  stream_exact<R, NT, LIMBS>(x, c, iters, total_waves, lane, a, ls);
  c += iters * total_waves;
  // the partial chain at the end: values past n read as +0.0
  const bool tail = c == chains_full && chains_full * R * kChunk < n;
  auto load_tail = [&](u32x4 (&v)[R]) {
    const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint64_t e = (c * R + r) * kChunk + uint64_t(lane) * 8;
      v[r] = e < n ? load8_masked(xh, e, n, 0u) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (tail) {
    u32x4 v[R];
    load_tail(v);
    if constexpr (LIMBS) {
      add_chain_limbs<R>(v, digit_selector(lane), ls);
    } else {
      add_chain<R>(v, a);
    }
  }
  if constexpr (LIMBS) {
    limbs_to_exact(ls, lane, (iters + (tail ? 1 : 0)) * R, a);
    // A wavefront that loaded an infinity or a NaN reads its chains again in
    // binary64 (add_chain) for the non-finite flags only: a set flag decides
    // the result and the integers are then not used.  Never taken on finite
    // data, so the stream above carries no such work.
    if (__builtin_amdgcn_ballot_w64(ls.expo == 31u) != 0) {
      Exact f{0, 0, 0};
      LimbSums unused{{0, 0, 0, 0}, 0};
      stream_exact<R, NT, false>(x, c0, iters, total_waves, lane, f, unused);
      if (tail) {
        u32x4 v[R];
        load_tail(v);
        add_chain<R>(v, f);
      }
      a.flags |= f.flags;
    }
  }
  fold(a);
  const Exact block_total = block_exact(wave_exact(a), lds);

  if (gridDim.x == 1) {
    if (threadIdx.x == 0) finish_exact(block_total, out, out_fixed);
    return;
  }
  const unsigned b = blockIdx.x, G = gridDim.x;
  const unsigned g = b / group, g0 = g * group;
  const unsigned in_group = G - g0 < group ? G - g0 : group;
  const unsigned groups = (G + group - 1) / group;
  if (!publish_with_ticket([&] { store_record(partials + uint64_t(b) * kRecordWords, block_total); },
                           counters + (1 + g) * kTicketStride, in_group, &flag))
    return;
  const Exact gv = combine_records(partials + uint64_t(g0) * kRecordWords, in_group, lds);
  if (groups == 1) {
    if (threadIdx.x == 0) finish_exact(gv, out, out_fixed);
    return;
  }
  __syncthreads();
  if (!publish_with_ticket([&] { store_record(group_partials + uint64_t(g) * kRecordWords, gv); },
                           counters, groups, &flag))
    return;
  const Exact v = combine_records(group_partials, groups, lds);
  if (threadIdx.x == 0) finish_exact(v, out, out_fixed);
}

// n == 0: out = +0.0, the 128-bit sum 0.
__global__ void exact_zero_kernel(float* out, int64_t* out_fixed) {
  if (threadIdx.x == 0) {
    out[0] = 0.0f;
    if (out_fixed) {
      out_fixed[0] = 0;
      out_fixed[1] = 0;
    }
  }
}

template <int R, bool LIMBS>
const void* pick_exact_nt(bool nt) {
  return nt ? reinterpret_cast<const void*>(&exact_kernel<R, true, LIMBS>)
            : reinterpret_cast<const void*>(&exact_kernel<R, false, LIMBS>);
}

template <int R>
const void* pick_exact(bool nt, bool limbs) {
  return limbs ? pick_exact_nt<R, true>(nt) : pick_exact_nt<R, false>(nt);
}

const void* exact_kernel_for(int r, bool nt, bool limbs) {
  switch (r) {
    case 1: return pick_exact<1>(nt, limbs);
    case 2: return pick_exact<2>(nt, limbs);
    case 3: return pick_exact<3>(nt, limbs);
    case 4: return pick_exact<4>(nt, limbs);
    case 5: return pick_exact<5>(nt, limbs);
    case 6: return pick_exact<6>(nt, limbs);
    case 7: return pick_exact<7>(nt, limbs);
    case 8: return pick_exact<8>(nt, limbs);
    default: return nullptr;
  }
}

}  // namespace

hipError_t launch_exact(const Plan& plan, const void* x, float* out, int64_t* out_fixed,
                        void* ws, hipStream_t stream) {
  if (plan.n == 0) {
    void* args[] = {&out, &out_fixed};
    return hipLaunchKernel(reinterpret_cast<const void*>(&exact_zero_kernel), dim3(1), dim3(64),
                           args, 0, stream);
  }
  const void* fn = exact_kernel_for(plan.r, (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0,
                                    (plan.flags & ARMX_FLAG_INT_LIMBS) != 0);
  if (!fn) return hipErrorInvalidValue;
  const u32x4* xv = static_cast<const u32x4*>(x);
  uint64_t n = plan.n;
  uint64_t chains_full = n / (uint64_t(plan.r) * kChunk);
  char* base = static_cast<char*>(ws);
  unsigned* counters = reinterpret_cast<unsigned*>(base);
  uint64_t* partials = reinterpret_cast<uint64_t*>(base + kCounterBytes);
  uint64_t* group_partials = reinterpret_cast<uint64_t*>(base + kCounterBytes + plan.partials_bytes);
  unsigned group = plan.group;
  void* args[] = {&xv, &n, &chains_full, &counters, &partials, &group_partials, &group, &out,
                  &out_fixed};
  return launch_main(plan, fn, args, stream);
}

}  // namespace armx
