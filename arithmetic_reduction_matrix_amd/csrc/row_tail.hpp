// Rows that end inside a chain, for the pipelined row streams
// (rows_kernels.hip, rows_fixed_kernels.hip): reading and masking a row's
// last chain.
#pragma once

#include "device_common.hpp"

namespace armx {
namespace dev {

// ---- rows that end inside a chain --------------------------------------------
//
// A row-major matrix of `rows` rows of `cols` values (cols > 512) with pitch
// ld >= cols, a multiple of 8 when there is more than one row, so every row
// starts 16-byte aligned.  The chunk grid restarts at every row, and a row's
// last chain of R chunks may end inside the row's last chunk or before it.
// The row streams read such a chain with load_row_chain_range, which fetches
// nothing past the row's last 16-byte lane slot.  In the plain form
// (load_row_chain), chunks past the row's last chunk are read from
// kNegZeroChunk, 1 KiB of -0.0 that stays in the caches (rereading the row's
// own last chunk instead costs HBM traffic: non-temporal loads do not keep
// it); -0.0 adds nothing in either order; and in the last chunk the lanes
// past the row read on into the pitch and the next row: at most 511 values
// past the row, so inside the matrix for every row but the last (the next
// row starts at most ld values on and holds more than 512).  The range-checked
// form reads the partly filled slot whole, inside the pitch, so it too may
// not read the matrix's last row: the pipelined streams read the last chain
// of that row apart, with load_last_chain, and the values of a last chain
// that are not the row's are replaced by `fill` in registers.
struct NegZeroChunk {
  uint32_t w[256];
  constexpr NegZeroChunk() : w() {
    for (int i = 0; i < 256; ++i) w[i] = 0x80008000u;
  }
};
// Never written.  Not const, and with external (inline) linkage, so that the
// optimiser cannot fold its contents into the loads that may read it: it
// would turn them into selects and branches, and the loop would no longer
// keep every load unconditional.
__device__ inline NegZeroChunk kNegZeroChunk{};

__device__ __forceinline__ const u32x4* neg_zero_chunk() {
  return reinterpret_cast<const u32x4*>(kNegZeroChunk.w);
}

// Loads chain c of the row at xr (R chunks, 16 bytes per lane each); chunks
// past `last_chunk` are read from `fill` (neg_zero_chunk()).
template <int R, bool NT>
__device__ __forceinline__ void load_row_chain(const uint16_t* __restrict__ xr, uint64_t c,
                                               uint64_t last_chunk, const u32x4* fill, int lane,
                                               u32x4 (&v)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint64_t ci = c * R + uint64_t(r);
    const u32x4* p = ci <= last_chunk ? reinterpret_cast<const u32x4*>(xr) + ci * 64 : fill;
    v[r] = load16<NT>(p + lane);
  }
}

// load_row_chain through a range-checked buffer descriptor over the row's
// first `row_bytes` bytes (its cols values rounded up to whole 16-byte lane
// slots): a lane whose slot starts at or past that end reads zeros without
// any memory access, so the lanes past the row in its last chunk, and chunks
// wholly past it, cost no fetch (with plain loads they read on into the next
// row, which a non-temporal stream then fetches from HBM a second time).
// Offsets are 32-bit: rows of less than 4 GiB.  The values past cols are
// replaced by the masks of row_tail_keep as before.
constexpr int kBufferWord3 = 0x00020000;   // raw buffer: 32-bit data, range-checked
template <int R, bool NT>
__device__ __forceinline__ void load_row_chain_range(const uint16_t* __restrict__ xr,
                                                     uint32_t row_bytes, uint64_t c, int lane,
                                                     u32x4 (&v)[R]) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xr), 0, int(row_bytes), kBufferWord3);
  const uint32_t off = uint32_t(c) * uint32_t(R) * 1024u + uint32_t(lane) * 16u;
#pragma unroll
  for (int r = 0; r < R; ++r)
    v[r] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + uint32_t(r) * 1024u, 0, NT ? 2 : 0));
}

// load_row_chain with the chain's chunks inside the row counted once per
// chain, in 32 bits (a row holds fewer than 2^31 chunks), so that choosing
// each chunk's address is a scalar compare and select.  PARTIAL false: rows
// are whole chains, so no chunk lies past the row and none is checked.
// (Measured against load_row_chain: faster in the fixed-order stream, 3992
// values 77.5 -> 76.4 us, and slower in the free-order stream of short rows,
// so each stream keeps the form that measured faster in it.)
template <int R, bool NT, bool PARTIAL>
__device__ __forceinline__ void load_row_chain_counted(const uint16_t* __restrict__ xr,
                                                       uint64_t c, uint64_t last_chunk,
                                                       const u32x4* fill, int lane,
                                                       u32x4 (&v)[R]) {
  const u32x4* base = reinterpret_cast<const u32x4*>(xr) + c * R * 64;
  if constexpr (!PARTIAL) {
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = load16<NT>(base + r * 64 + lane);
  } else {
    const uint32_t left = uint32_t(last_chunk + 1 - c * R);
    const uint32_t inside = left < uint32_t(R) ? left : uint32_t(R);
#pragma unroll
    for (int r = 0; r < R; ++r)
      v[r] = load16<NT>((uint32_t(r) < inside ? base + r * 64 : fill) + lane);
  }
}

// Replaces the values of chain c (as loaded by load_row_chain) at or past
// cols by `fill` (a binary16 pattern).  Applied to all-ones registers it
// gives the masks of row_tail_keep.
template <int R>
__device__ __forceinline__ void mask_row_chain(u32x4 (&v)[R], uint64_t c, uint64_t cols,
                                               uint32_t fill, int lane) {
  const uint32_t f2 = fill | (fill << 16);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint64_t cs = (c * R + uint64_t(r)) * 512;
    const uint64_t in_chunk = cs >= cols ? 0 : (cols - cs > 512 ? 512 : cols - cs);
    const int left = int(in_chunk) - lane * 8;   // values of this lane's slot in the row
    const int k = left < 0 ? 0 : (left > 8 ? 8 : left);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t keep = (2 * w < k ? 0xFFFFu : 0u) | (2 * w + 1 < k ? 0xFFFF0000u : 0u);
      v[r][w] = (v[r][w] & keep) | (f2 & ~keep);
    }
  }
}

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

// The last chain of the matrix's last row, which the pipelined loads may not
// read past, read with no read past the row's cols values and no branch
// around a load, in two steps so that the loads can be issued long before
// the values are needed.  load_last_chain issues them: lanes whose 8 values
// lie inside the row load them, the others read the -0.0 chunk (those
// values are masked by apply_row_tail); when the row ends inside a lane's 8
// values, every lane also reads those values one by one (clamped to the
// row) into h.  merge_last_chain then gives that lane its values.  The
// caller applies the masks of row_tail_keep.
template <int R, bool NT>
__device__ __forceinline__ void load_last_chain(const uint16_t* __restrict__ xr, uint64_t c,
                                                uint64_t cols, int lane, u32x4 (&v)[R],
                                                uint32_t (&h)[8]) {
  const u32x4* fill = neg_zero_chunk() + lane;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint64_t e = (c * R + uint64_t(r)) * 512 + uint64_t(lane) * 8;
    v[r] = load16<NT>(e + 8 <= cols ? reinterpret_cast<const u32x4*>(xr + e) : fill);
  }
  const uint64_t es = cols & ~uint64_t(7);   // the 8 values the row ends inside
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = xr[es + uint64_t(i) < cols ? es + uint64_t(i) : cols - 1];
}

template <int R>
__device__ __forceinline__ void merge_last_chain(u32x4 (&v)[R], const uint32_t (&h)[8],
                                                 uint64_t c, uint64_t cols, int lane) {
  const uint64_t es = cols & ~uint64_t(7);
  if (es == cols) return;   // the row ends at a lane boundary
  const u32x4 w{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                h[6] | (h[7] << 16)};
  const uint64_t rs = es / 512 - c * R, ls = (es % 512) / 8;
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = (uint64_t(r) == rs && uint64_t(lane) == ls) ? w : v[r];
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
