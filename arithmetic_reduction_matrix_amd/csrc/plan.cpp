// Argument checking and launch planning (host only, no HIP calls).
#include "plan.h"

#include <cmath>
#include <initializer_list>

namespace armx {
namespace {

constexpr unsigned kKnownFlags = ARMX_FLAG_PLAIN | ARMX_FLAG_CACHED_LOADS |
                                 ARMX_FLAG_ONE_CHAIN | ARMX_FLAG_TWO_PASS |
                                 ARMX_FLAG_MMA_LEVELS | ARMX_FLAG_MMA_LEAVES |
                                 ARMX_FLAG_ALL_ONES | ARMX_FLAG_INT_LIMBS;

uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

bool is_pow2(uint64_t v) { return v && !(v & (v - 1)); }

int log2_ceil(uint64_t v) {
  int k = 0;
  while ((uint64_t(1) << k) < v) ++k;
  return k;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int log2_floor(uint64_t v) {
  int k = 0;
  while (v > 1) {
    v >>= 1;
    ++k;
  }
  return k;
}

// Whether `blocks` blocks spread evenly over the compute units.
bool even_blocks(uint64_t blocks, int cu_count) {
  return blocks <= uint64_t(cu_count) || blocks % uint64_t(cu_count) == 0;
}

// Wavefronts per block of a split (mode 3) with an automatic block size: the
// part count over the compute-unit count, rounded up (1 to kMaxWaves), so
// that no compute unit gets a second block -- measured on MI355X, a grid a
// little larger than the compute-unit count finishes when its doubly loaded
// units do, up to half again as late.
uint64_t split_block(uint64_t items, int cu_count) {
  uint64_t w = ceil_div(items, uint64_t(cu_count));
  if (w < 1) w = 1;
  if (w > uint64_t(kMaxWaves)) w = uint64_t(kMaxWaves);
  return w;
}

// Blocks of W wavefronts an automatic persistent grid uses: about
// loads_per_cu / R wavefronts per compute unit, at least one block per unit.
uint64_t persistent_blocks(const OpDefaults& d, int cu_count, uint64_t W, uint64_t R) {
  const uint64_t waves_per_cu = (uint64_t(d.loads_per_cu) + R - 1) / R;
  uint64_t blocks = uint64_t(cu_count) * waves_per_cu / W;
  if (blocks < uint64_t(cu_count)) blocks = uint64_t(cu_count);
  return blocks;
}

// Automatic grids for flat reductions of small inputs: a call costs about
// a n / g (streaming per wavefront) + b g (block launch and completion ticket)
// for g wavefronts, smallest near g ~ sqrt(n).  A wavefront streams R loads
// per step, so the cap is sqrt(n) / R wavefronts; measured on MI355X at R = 8
// (64 blocks of 2 at n = 2^20) it is within a few percent of the best grid
// from 2^18 to 2^24 for the free-order, fixed-order and exact sums.  It only
// applies below the persistent grid's own target (loads_per_cu / R
// wavefronts per compute unit), so large inputs keep the full persistent grid
// whatever the block size.  Returns `blocks` or the smaller capped count.
uint64_t cap_small_input(uint64_t blocks, uint64_t n, const OpDefaults& d, int cu_count,
                         uint64_t W, uint64_t R) {
  const uint64_t cap_waves = uint64_t(std::ceil(std::sqrt(double(n)) / double(R)));
  const uint64_t target_waves = uint64_t(cu_count) * ((uint64_t(d.loads_per_cu) + R - 1) / R);
  if (cap_waves >= target_waves) return blocks;
  uint64_t cap = (cap_waves + W - 1) / W;
  if (cap < 1) cap = 1;
  return blocks < cap ? blocks : cap;
}

// Rows of at most one chunk (mode 2): a row takes ceil(cols / 8) lanes,
// padded to a power of two.  Staged widths: the rows (all but a last row
// whose width is not a multiple of 8, which one wavefront sums apart) are cut
// into chunks of whole steps, about one per block of the persistent grid and
// at most kShortChunkRows rows, which the blocks take in turn.  Sets the mode,
// the lane count, the groups per step (r), the grid and, when staged, the
// chunk and its LDS.
void plan_short_rows(Plan& p, int cu_count, uint64_t W, int grid_cap) {
  const uint64_t lanes = (p.n + 7) / 8;
  int lg = 0;
  while ((uint64_t(1) << lg) < lanes) ++lg;
  p.mode = 2;
  p.seg_log2 = lg;
  const bool staged = lg >= kShortStagedMinLog2;
  p.r = staged && (p.rows == 1 || p.ld % 64 == 0) ? 4 : 8;   // groups per step
  const uint64_t rows_per_step = (uint64_t(64) >> lg) * uint64_t(p.r);
  uint64_t target = ceil_div(uint64_t(cu_count) * kShortWavesPerCu, W);
  if (grid_cap > 0 && target > uint64_t(grid_cap)) target = uint64_t(grid_cap);
  if (staged) p.xcd_remap = 0;   // a chunk is one block's range of rows already
  if (!staged) {
    const uint64_t waves = ceil_div(p.rows, rows_per_step);
    const uint64_t grid = ceil_div(waves, W);
    p.grid = int(grid < 1 ? 1 : (grid < target ? grid : target));
    p.chunk_rows = 0;
    p.lds_bytes = 0;
    return;
  }
  const uint64_t body = p.rows - (p.n % 8 ? 1 : 0);
  uint64_t per_chunk = ceil_div(ceil_div(body, rows_per_step), target);
  if (per_chunk < 1) per_chunk = 1;
  if (per_chunk > kShortChunkRows / rows_per_step) per_chunk = kShortChunkRows / rows_per_step;
  p.chunk_rows = per_chunk * rows_per_step;
  const uint64_t chunks = ceil_div(body, p.chunk_rows);
  const uint64_t grid = chunks < target ? chunks : target;
  p.grid = int(grid < 1 ? 1 : grid);
  p.lds_bytes = size_t(p.chunk_rows) * sizeof(float);
}

// Automatic shapes for rows longer than one chunk (cols > 512), measured on
// MI355X with 2^28 values.  A row stream keeps two chains in flight per
// wavefront whatever they hold, so a row's last chain should be as full as
// possible: one that holds a single chunk costs about as long as a full one
// (9-chunk rows at R = 8: 111 us against 77 us at R = 5).
//  * Rows of fewer than 8 chunks carry a fixed cost per row (the chain's
//    result, the row combine, the store) that more wavefronts hide: R = 1
//    (16 wavefronts per compute unit) in blocks of 512 threads, except free-
//    order rows of 4, 6 or 7 chunks in matrices of at least four rounds of
//    that stream, which take R = 2 (half the chains per row, the same loads
//    in flight; 2600-value rows 88.0 -> 83.1 us, 2048 79.1 -> 77.7, 3072
//    78.9 -> 77.3, 3200 86.1 -> 81.4, 3584 79.2 -> 76.6; 2-chunk rows lose,
//    79.9 -> 97.6 us, 3-chunk rows gain or lose by width, and small matrices
//    lose, 1500 x 2048 4.1 -> 4.5 us), and of 5 chunks, which take R = 3 in
//    blocks of 64 (2456 values 82.3 -> 80.3 us, 2260 87.0 -> 84.6, 2560 78.2
//    -> 77.4).  Fixed order: rows of exactly 2 or 4 chunks are one group each
//    (R = chunks; 4 chunks in blocks of 256 in such matrices, 80.9 -> 74.8
//    us), other rows of 2, 4 or 6 chunks in such matrices R = 2 in blocks of
//    256 (2600 values 95.8 -> 87.2 us, 3072 78.9 -> 75.9, 920 89.7 -> 83.5,
//    1000 82.0 -> 79.1), rows of 7 chunks R = 4 in blocks of 256 (3480
//    values 85.5 -> 81.3 us, 3284 89.7 -> 85.3), other short rows R = 1 in
//    blocks of 256.
//  * Longer fixed-order rows: the R of 2 and 4 that pads the last group
//    least (R = 2 only while a row stays within the flat kernel's 64
//    groups), 4 on a tie, default blocks.
//  * Longer free-order rows, default blocks.  8 to 13 chunks: the R of 8, 5
//    and 4 that pads the last chain least, the larger on a tie, except that
//    rows of 8 chunks ending inside the last one take R = 4 (such a row is
//    one masked chain at R = 8, two wavefronts per compute unit, and streams
//    slower than a whole one: 3992 values 87.9 us at R = 8, 77.6 at R = 4,
//    where 4096 values run 74.2 us at R = 8).  14 chunks or more: R = 8
//    when the padding of its last chain is at most a fifth of the row and,
//    below 22 chunks (at most three chains of 8), at most one chunk; else
//    R = 4.  Measured over 23 lengths from 14 to 64 chunks this is within
//    about 1 us of the better of R = 4 and 8 (22 chunks 76.7 us at R = 8
//    against 77.6 at R = 4, 20 chunks 79.9 against 77.3, 25 chunks 80.5
//    against 77.3, 50 chunks 77.3 against 80.5); R = 5 pads less in some of
//    these and is never measurably faster than that better one (20 chunks
//    78.2 us, 25 chunks 78.8).  Free order skips R = 6
//    and 7: their grids hold 3 wavefronts per compute unit, which streamed
//    rows measurably worse (768 rows of 348712 values: 97.4 us at R = 6
//    against 78.7 us at R = 4; over 24 row counts at 2^28 values the slowest
//    shape went from 1.24 to 1.08 times its best R).
struct RowShape {
  uint64_t r;
  int block;
};

RowShape rows_auto_shape(uint64_t rows, uint64_t cols, int cu_count, const OpDefaults& d,
                         bool fixed) {
  const uint64_t chunks = ceil_div(cols, kChunk);
  if (chunks < 8) {
    // (the other R only with rows for four rounds of the R = 1 stream:
    // smaller matrices are latency-bound and want the wavefronts)
    const bool many = rows >= 4 * 16 * uint64_t(cu_count);
    if (fixed) {
      if (chunks == 4 && cols == chunks * kChunk) return {4, many ? 256 : 512};
      if (chunks == 2 && cols == chunks * kChunk) return {2, 512};
      if (many && (chunks == 2 || chunks == 4 || chunks == 6)) return {2, 256};
      if (many && chunks == 7) return {4, 256};
      return {1, 256};
    }
    if (many && (chunks == 4 || chunks == 6 || chunks == 7)) return {2, 512};
    if (many && chunks == 5) return {3, 64};
    return {1, 512};
  }
  auto waste = [&](uint64_t r) { return ceil_div(chunks, r) * r - chunks; };
  if (fixed) {
    const uint64_t r = (waste(2) < waste(4) && ceil_div(chunks, 2) <= 64) ? 2 : 4;
    return {r, d.block};
  }
  if (chunks >= 14) {
    const uint64_t w8 = waste(8);
    const bool r8 = 5 * w8 <= chunks && (chunks >= 22 || w8 <= 1);
    return {r8 ? uint64_t(8) : uint64_t(4), d.block};
  }
  if (chunks == 8 && cols % kChunk != 0) return {4, d.block};
  uint64_t best = 8;
  for (uint64_t r : {uint64_t(5), uint64_t(4)})
    if (waste(r) < waste(best)) best = r;
  return {best, d.block};
}

// Consecutive rows whose pitch is not a whole number of 128-byte lines share
// a line; with blocks dispatched round-robin over the XCDs, each XCD would
// fetch it.  Such rows get the XCD-contiguous block order.  (Measured on
// MI355X: 1000-value rows 85 -> 78 us; rows of whole lines gain nothing and
// 4096-value rows lose, 74 -> 79 us.)
int rows_remap(uint64_t rows, uint64_t ld) { return rows > 1 && ld % 64 != 0 ? 1 : 0; }

// Ticket groups.  Up to kSingleLevelMax blocks use one group: the tail of
// the kernel then has the fewest serialised memory round trips (measured
// faster at 256 blocks).  Larger grids use a power-of-two group size near
// sqrt(grid), so that neither a group counter nor the top counter sees many
// increments, with at most kMaxGroups groups (measured on MI355X, 2^28
// values, 64-thread blocks: at R = 4, 1024 blocks, 86.0 us in one group and
// 76.9 us in 32; one chain per wavefront at R = 1, 2^19 blocks, 1848 us in 63
// groups and 619 us in 255).  Sets the workspace sizes.
constexpr uint64_t kSingleLevelMax = 256;

void size_ticket(Plan& p, size_t record_bytes = sizeof(float)) {
  const uint64_t G = uint64_t(p.grid);
  uint64_t group = 1;
  if (G <= kSingleLevelMax) {
    while (group < G) group <<= 1;
  } else {
    while (group * group < G) group <<= 1;
    while ((G + group - 1) / group > kMaxGroups) group <<= 1;
  }
  p.group = unsigned(group);
  p.partials_bytes = round_up(record_bytes * size_t(G), 256);
  p.ws_bytes = kCounterBytes + p.partials_bytes + round_up(record_bytes * kMaxGroups, 256);
}

}  // namespace

int make_plan(int op, uint64_t n_or_rows, uint64_t cols, uint64_t ld,
              const armx_config* cfg, int cu_count, Plan* plan, bool allow_split,
              bool split_in_halves) {
  armx_config c{};
  if (cfg) c = *cfg;
  const bool auto_r = c.chain_r == 0;
  const bool auto_block = c.block_threads == 0;
  const OpDefaults d = op == kOpFixed                    ? kFixedDefaults
                       : op == kOpRows                   ? kRowsDefaults
                       : op == kOpRowsFixed              ? kRowsFixedDefaults
                       : op == kOpExact && (c.flags & ARMX_FLAG_INT_LIMBS) ? kExactLimbsDefaults
                       : op == kOpExact                  ? kExactDefaults
                       : (c.flags & ARMX_FLAG_MMA_LEVELS) ? kLevelsDefaults
                                                         : kSumDefaults;
  if (c.block_threads == 0) c.block_threads = d.block;
  if (c.chain_r == 0) c.chain_r = d.r;
  if (c.block_threads < 64 || c.block_threads > 64 * kMaxWaves || c.block_threads % 64)
    return ARMX_ERR_CONFIG;
  if (c.chain_r < 1 || c.chain_r > kMaxR) return ARMX_ERR_CONFIG;
  if (c.grid_blocks < 0) return ARMX_ERR_CONFIG;
  if (c.flags & ~kKnownFlags) return ARMX_ERR_CONFIG;
  if (cu_count <= 0) cu_count = 256;

  Plan p;
  p.op = op;
  p.waves = c.block_threads / 64;
  p.r = c.chain_r;
  p.flags = c.flags;
  p.start_event = c.start_event;
  p.stop_event = c.stop_event;
  const uint64_t W = uint64_t(p.waves);
  uint64_t R = uint64_t(p.r);

  if (op != kOpSum && (c.flags & ARMX_FLAG_MMA_LEVELS)) return ARMX_ERR_CONFIG;
  if (op != kOpFixed && op != kOpRowsFixed && (c.flags & ARMX_FLAG_MMA_LEAVES))
    return ARMX_ERR_CONFIG;
  if (op != kOpExact && (c.flags & ARMX_FLAG_INT_LIMBS)) return ARMX_ERR_CONFIG;
  // the all-ones operand is a choice of the free-order MFMA design only
  if ((c.flags & ARMX_FLAG_ALL_ONES) &&
      ((op != kOpSum && op != kOpRows) ||
       (c.flags & (ARMX_FLAG_PLAIN | ARMX_FLAG_MMA_LEVELS))))
    return ARMX_ERR_CONFIG;
  if (op == kOpExact) {
    // persistent grid as for the free-order sum; the load kind and the
    // integer-limb form are the only flags
    if (c.flags & ~unsigned(ARMX_FLAG_CACHED_LOADS | ARMX_FLAG_INT_LIMBS)) return ARMX_ERR_CONFIG;
    if ((c.flags & ARMX_FLAG_INT_LIMBS) && p.waves > kExactLimbsMaxBlock / 64)
      p.waves = kExactLimbsMaxBlock / 64;
    const uint64_t W = uint64_t(p.waves);
    const uint64_t n = n_or_rows;
    if (n > kMaxN) return ARMX_ERR_SHAPE;
    p.n = n;
    if (n == 0) { *plan = p; return ARMX_OK; }
    const uint64_t chains = ceil_div(n, kChunk * R);
    uint64_t grid = ceil_div(chains, W);
    const uint64_t resident =
        cap_small_input(persistent_blocks(d, cu_count, W, R), n, d, cu_count, W, R);
    if (grid > resident) grid = resident;
    if (c.grid_blocks > 0 && grid > uint64_t(c.grid_blocks)) grid = uint64_t(c.grid_blocks);
    if (grid < 1) grid = 1;
    p.grid = int(grid);
    size_ticket(p, kExactRecordBytes);
  } else if (op == kOpSum) {
    const uint64_t n = n_or_rows;
    if ((c.flags & ARMX_FLAG_MMA_LEVELS) && (c.flags & (ARMX_FLAG_PLAIN | ARMX_FLAG_TWO_PASS)))
      return ARMX_ERR_CONFIG;
    if (n > kMaxN) return ARMX_ERR_SHAPE;
    p.n = n;
    if (n == 0) { *plan = p; return ARMX_OK; }
    const uint64_t chains = ceil_div(n, kChunk * R);
    uint64_t grid = ceil_div(chains, W);
    if (!(c.flags & ARMX_FLAG_ONE_CHAIN)) {
      const uint64_t resident =
          cap_small_input(persistent_blocks(d, cu_count, W, R), n, d, cu_count, W, R);
      if (grid > resident) grid = resident;
    }
    if (c.grid_blocks > 0 && grid > uint64_t(c.grid_blocks)) {
      if (c.flags & ARMX_FLAG_ONE_CHAIN) return ARMX_ERR_CONFIG;  // would not be one chain
      grid = uint64_t(c.grid_blocks);
    }
    if (grid < 1) grid = 1;
    if (grid > 0x7FFFFFFFull) return ARMX_ERR_SHAPE;
    p.grid = int(grid);
    if (c.flags & ARMX_FLAG_MMA_LEVELS) {
      // level buffers: level 1's values, then level 2's (levels 3, 4, ...
      // reuse them in turn); nothing when level 1 already gives one value
      const uint64_t c1 = level_count(n, R, 1);
      const uint64_t c2 = level_count(c1, R, 2);
      if (c1 > 1) {
        p.partials_bytes = round_up(sizeof(float) * size_t(c1), 256);
        p.aux_bytes = c2 > 1 ? round_up(sizeof(float) * size_t(c2), 256) : 0;
        p.ws_bytes = kCounterBytes + p.partials_bytes + p.aux_bytes;
      }
    } else {
      size_ticket(p);
    }
  } else if (op == kOpFixed) {
    const uint64_t n = n_or_rows;
    if (n > kMaxN) return ARMX_ERR_SHAPE;
    if (!is_pow2(W)) return ARMX_ERR_CONFIG;
    if (c.flags & (ARMX_FLAG_PLAIN | ARMX_FLAG_ONE_CHAIN)) return ARMX_ERR_CONFIG;
    p.n = n;
    if (n == 0) { *plan = p; return ARMX_OK; }
    const uint64_t chunks = ceil_div(n, kChunk);
    uint64_t target = cap_small_input(persistent_blocks(d, cu_count, W, R), n, d, cu_count, W, R);
    if (c.grid_blocks > 0 && target > uint64_t(c.grid_blocks)) target = uint64_t(c.grid_blocks);
    if (target > uint64_t(kFixedMaxBlocks)) target = kFixedMaxBlocks;
    if (target < 1) target = 1;
    // every wavefront owns an aligned power-of-two range of chunks, so every
    // wavefront and every block covers a complete subtree of the tree
    int lc = log2_ceil(ceil_div(chunks, W * target));
    // each wavefront logs one node per R-chunk group (power-of-two R) or per
    // chunk into LDS, in rows of 64: keep that within kFixedLdsBytes per
    // block by giving each wavefront fewer chunks (a larger grid)
    const uint64_t per_node = is_pow2(R) ? R : 1;
    auto slots = [&](int l) {
      uint64_t nodes = ceil_div(uint64_t(1) << l, per_node);
      return (nodes + 63) / 64 * 64;
    };
    while (lc > 0 && W * slots(lc) * sizeof(float) > kFixedLdsBytes) --lc;
    if (lc > kFixedMaxLog2Chunks) return ARMX_ERR_SHAPE;
    p.log2_chunks = lc;
    p.slots_per_wave = unsigned(slots(lc));
    p.lds_bytes = size_t(W) * slots(lc) * sizeof(float);
    const uint64_t grid = ceil_div(chunks, W << lc);
    if (grid > uint64_t(kFixedMaxBlocks)) return ARMX_ERR_SHAPE;
    p.grid = int(grid);
    size_ticket(p);
  } else if (op == kOpRows) {
    if (c.flags & (ARMX_FLAG_ONE_CHAIN | ARMX_FLAG_TWO_PASS)) return ARMX_ERR_CONFIG;
    const uint64_t rows = n_or_rows;
    if (ld < cols) return ARMX_ERR_SHAPE;
    if (cols > kMaxN || rows > kMaxN || (rows > 0 && ld > kMaxN / rows)) return ARMX_ERR_SHAPE;
    if (rows > 1 && cols > 0 && ld % 8) return ARMX_ERR_ALIGN;
    p.rows = rows;
    p.n = cols;
    p.ld = ld;
    p.xcd_remap = rows_remap(rows, ld);
    if (rows > 0 && cols > 0 && cols <= kChunk) {
      if (auto_block) p.waves = kShortBlock / 64;
      plan_short_rows(p, cu_count, uint64_t(p.waves), c.grid_blocks);
      p.ws_bytes = 0;
      *plan = p;
      return ARMX_OK;
    }
    uint64_t W = uint64_t(p.waves);
    if (cols > kChunk) {
      const RowShape a = rows_auto_shape(rows, cols, cu_count, d, false);
      if (auto_r) R = a.r;
      if (auto_block) W = uint64_t(a.block / 64);
      p.r = int(R);
      p.waves = int(W);
    }
    // many rows: one wavefront per row over a persistent grid; few rows:
    // each row split over wavefronts of several blocks (mode 3, with a
    // workspace) or, without one, a block per row so that every row still
    // gets W wavefronts
    const uint64_t blocks = persistent_blocks(d, cu_count, W, R);
    const uint64_t waves = blocks * W;
    uint64_t grid;
    // A row stream whose last round of rows is poorly filled (under 90%,
    // within four rounds) finishes with most wavefronts idle: with a
    // workspace, such rows are split in two instead, every half row a
    // wavefront of its own, all resident at once when the halves fit 16
    // per compute unit (measured on MI355X, 2^28 values: 900 rows 99.8 ->
    // 82.1 us, 1200 rows 99.2 -> 84.8 us).
    // (grid_blocks is an upper bound on the grid: a split that would need
    // more blocks is not planned.)
    const uint64_t rounds = ceil_div(rows, waves);
    const uint64_t W_halves = split_block(rows * 2, cu_count);
    if (allow_split && auto_block && rows >= waves && rows < 4 * waves &&
        10 * rows < 9 * rounds * waves && 2 * rows <= uint64_t(kMaxWaves) * uint64_t(cu_count) &&
        cols >= 2 * kSplitMinSegment &&
        (c.grid_blocks == 0 || ceil_div(rows * 2, W_halves) <= uint64_t(c.grid_blocks))) {
      const uint64_t S = 2, W3 = W_halves;
      p.mode = 3;
      p.waves = int(W3);
      p.segs = unsigned(S);
      p.grid = int(ceil_div(rows * S, W3));
      p.partials_bytes = round_up(sizeof(float) * size_t(rows * S), 256);
      p.ws_bytes = kCounterBytes + p.partials_bytes;
      *plan = p;
      return ARMX_OK;
    }
    if (rows >= waves) {
      p.mode = 1;
      grid = blocks;
      if (grid > ceil_div(rows, W)) grid = ceil_div(rows, W);
    } else {
      p.mode = 0;
      grid = rows;
      const uint64_t cpr = ceil_div(cols, R * kChunk);   // chains per row
      if (allow_split && rows > 0 && 4 * rows * W < 3 * waves && cols / W >= kSplitMinShare) {
        // the row's chains are dealt round-robin to its S wavefronts; S
        // rounds the grid's wavefront count per row down, so that the parts
        // fit that count and the blocks cover the compute units (rounding up
        // gave rows x S just over it, three wavefronts per block and blocks
        // on two thirds of the units: 2^28 values, 20 rows 87.5 -> 79.8 us,
        // 13 rows 86.5 -> 79.5, 3 rows 80.4 -> 77.1, 250 rows 85.9 -> 81.7;
        // 200 rows 85.8 -> 86.2)
        uint64_t S = waves / rows >= 2 ? waves / rows : ceil_div(waves, rows);
        S = S < cpr ? S : cpr;
        S = S < cols / kSplitMinSegment ? S : cols / kSplitMinSegment;
        S = S < kSplitMaxSegs ? S : kSplitMaxSegs;   // what the last block's tree holds
        const uint64_t W3 = auto_block ? split_block(rows * S, cu_count) : W;
        uint64_t cap = kSplitMaxBlocks;
        if (c.grid_blocks > 0 && uint64_t(c.grid_blocks) < cap) cap = uint64_t(c.grid_blocks);
        if (ceil_div(rows * S, W3) > cap) S = cap * W3 / rows;
        if (S >= 2) {
          p.mode = 3;
          p.waves = int(W3);
          p.segs = unsigned(S);
          p.grid = int(ceil_div(rows * S, W3));
          p.partials_bytes = round_up(sizeof(float) * size_t(rows * S), 256);
          p.ws_bytes = kCounterBytes + p.partials_bytes;
          *plan = p;
          return ARMX_OK;
        }
      }
      // a block per row (no workspace); with an automatic block size, rows
      // that give the persistent grid's wavefront count less than three
      // quarters get about that count's share each (any W: the row's chains
      // are dealt round-robin; at most one wavefront per chain) -- when the
      // blocks spread evenly over the compute units (measured on MI355X:
      // wider blocks on a grid a little larger than the unit count lose)
      if (auto_block && rows > 0 && even_blocks(rows, cu_count) && 4 * rows * W < 3 * waves) {
        uint64_t w = ceil_div(waves, rows);
        if (w > cpr) w = cpr;
        if (w > uint64_t(kMaxWaves)) w = uint64_t(kMaxWaves);
        if (w > W) W = w;
        p.waves = int(W);
      }
    }
    if (grid > (uint64_t(1) << 20)) grid = uint64_t(1) << 20;   // blocks loop over rows
    if (c.grid_blocks > 0 && grid > uint64_t(c.grid_blocks)) grid = uint64_t(c.grid_blocks);
    if (grid < 1) grid = 1;
    p.grid = int(grid);
    p.ws_bytes = 0;
  } else if (op == kOpRowsFixed) {
    if (c.flags & (ARMX_FLAG_PLAIN | ARMX_FLAG_ONE_CHAIN | ARMX_FLAG_TWO_PASS))
      return ARMX_ERR_CONFIG;
    if (!is_pow2(W)) return ARMX_ERR_CONFIG;
    const uint64_t rows = n_or_rows;
    if (ld < cols) return ARMX_ERR_SHAPE;
    if (cols > kMaxN || rows > kMaxN || (rows > 0 && ld > kMaxN / rows)) return ARMX_ERR_SHAPE;
    if (rows > 1 && cols > 0 && ld % 8) return ARMX_ERR_ALIGN;
    p.rows = rows;
    p.n = cols;
    p.ld = ld;
    if (rows == 0 || cols == 0) { *plan = p; return ARMX_OK; }
    p.xcd_remap = rows_remap(rows, ld);
    if (cols <= kChunk) {
      if (auto_block) p.waves = kShortBlock / 64;
      if ((c.flags & ARMX_FLAG_MMA_LEAVES) && p.waves > kShortMmaMaxBlock / 64)
        p.waves = kShortMmaMaxBlock / 64;
      plan_short_rows(p, cu_count, uint64_t(p.waves), c.grid_blocks);
      *plan = p;
      return ARMX_OK;
    }
    uint64_t W = uint64_t(p.waves);
    {
      const RowShape a = rows_auto_shape(rows, cols, cu_count, d, true);
      if (auto_r) R = a.r;
      if (auto_block) W = uint64_t(a.block / 64);
      p.r = int(R);
      p.waves = int(W);
    }
    uint64_t blocks = persistent_blocks(d, cu_count, W, R);
    const uint64_t group_elems = R * kChunk;
    bool flat = is_pow2(R) && ceil_div(cols, group_elems) <= 64 && (rows >= blocks * W || W == 1);
    // Rows that give the persistent grid's wavefront count less than three
    // quarters: split each row into S aligned power-of-two chunk ranges
    // (subtrees), one wavefront each in blocks of W3; the last block's tree
    // over a row's S segment roots is the row's tree.  The range size is the
    // largest power of two that still gives at least the grid's wavefront
    // count of ranges in all, so no wavefront holds more than its share (a
    // row's last range may be short).  The ranges are long, so an automatic
    // R is the flat fixed-order sum's 8.
    const uint64_t per_row = flat ? 1 : W;
    const bool halves = allow_split && split_in_halves;
    if (allow_split &&
        (halves || (4 * rows * per_row < 3 * blocks * W && cols / per_row >= kSplitMinShare))) {
      const uint64_t R3 = auto_r ? uint64_t(kFixedDefaults.r) : R;
      const uint64_t waves3 = persistent_blocks(d, cu_count, 1, R3);
      const uint64_t chunks = ceil_div(cols, kChunk);
      const uint64_t per_node = is_pow2(R3) ? R3 : 1;
      auto segs_for = [&](int l) { return ceil_div(chunks, uint64_t(1) << l); };
      auto slots_for = [&](int l) {
        return (ceil_div(uint64_t(1) << l, per_node) + 63) / 64 * 64;
      };
      const int min_lc = log2_ceil(kSplitMinSegment / kChunk);
      int lc = rows * chunks >= waves3 ? log2_floor(rows * chunks / waves3) : 0;
      if (halves) lc = log2_ceil(ceil_div(chunks, 2));   // two ranges per row
      if (lc < min_lc) lc = min_lc;
      while (segs_for(lc) > kSplitMaxSegs || rows * segs_for(lc) > kSplitMaxItems) ++lc;
      const uint64_t W3 = auto_block ? split_block(rows * segs_for(lc), cu_count) : W;
      uint64_t cap = kSplitMaxBlocks;
      if (c.grid_blocks > 0 && uint64_t(c.grid_blocks) < cap) cap = uint64_t(c.grid_blocks);
      while (ceil_div(rows * segs_for(lc), W3) > cap && segs_for(lc) > 1) ++lc;
      // node logs, beside the last block's stage of parts: fewer chunks per
      // segment (more segments) while they do not fit
      const size_t log_bytes = kFixedLdsBytes - kSplitMaxItems * sizeof(float);
      while (W3 * slots_for(lc) * sizeof(float) > log_bytes && lc > min_lc &&
             segs_for(lc - 1) <= kSplitMaxSegs && ceil_div(rows * segs_for(lc - 1), W3) <= cap)
        --lc;
      const uint64_t S = segs_for(lc);
      if (S >= 2 && lc <= kFixedMaxLog2Chunks &&
          W3 * slots_for(lc) * sizeof(float) <= log_bytes) {
        p.mode = 3;
        p.r = int(R3);
        p.waves = int(W3);
        p.segs = unsigned(S);
        p.log2_chunks = lc;
        p.slots_per_wave = unsigned(slots_for(lc));
        p.lds_bytes = size_t(W3 * slots_for(lc) * sizeof(float));
        p.grid = int(ceil_div(rows * S, W3));
        p.partials_bytes = round_up(sizeof(float) * size_t(rows * S), 256);
        p.ws_bytes = kCounterBytes + p.partials_bytes;
        *plan = p;
        return ARMX_OK;
      }
    }
    // otherwise, with an automatic block size, rows that give the persistent
    // grid's wavefront count less than three quarters get more wavefronts
    // each (the general mapping, W per row; measured on MI355X, a fixed-order
    // wavefront at R = 4 keeps fewer bytes in flight than a free-order one)
    if (auto_block && rows < blocks * W && even_blocks(rows, cu_count)) {
      const uint64_t target = blocks * W, chunks = ceil_div(cols, kChunk);
      uint64_t W2 = W;
      while (4 * rows * W2 < 3 * target && 2 * W2 <= chunks && W2 < uint64_t(kMaxWaves)) W2 *= 2;
      if (W2 != W) {
        W = W2;
        p.waves = int(W);
        blocks = persistent_blocks(d, cu_count, W, R);
        flat = false;
      }
    }
    uint64_t grid;
    if (flat) {
      // flat: a wavefront's rows stream back to back; each row is at most
      // 64 group subtrees, one per lane of a slot register
      p.mode = 1;
      grid = blocks;
      if (grid > ceil_div(rows, W)) grid = ceil_div(rows, W);
    } else {
      // general: a block per row, W wavefronts on aligned power-of-two
      // chunk ranges, node logs in LDS
      p.mode = 0;
      const uint64_t chunks = ceil_div(cols, kChunk);
      const int lc = log2_ceil(ceil_div(chunks, W));
      const uint64_t per_node = is_pow2(R) ? R : 1;
      const uint64_t nodes = ceil_div(uint64_t(1) << lc, per_node);
      const uint64_t slots = (nodes + 63) / 64 * 64;
      if (W * slots * sizeof(float) > kFixedLdsBytes) return ARMX_ERR_SHAPE;
      p.log2_chunks = lc;
      p.slots_per_wave = unsigned(slots);
      p.lds_bytes = size_t(W * slots * sizeof(float));
      grid = rows;
    }
    if (grid > (uint64_t(1) << 20)) grid = uint64_t(1) << 20;   // blocks loop over rows
    if (c.grid_blocks > 0 && grid > uint64_t(c.grid_blocks)) grid = uint64_t(c.grid_blocks);
    if (grid < 1) grid = 1;
    p.grid = int(grid);
    p.ws_bytes = 0;
  } else {
    return ARMX_ERR_CONFIG;
  }
  *plan = p;
  return ARMX_OK;
}

int make_row_plans(int op, uint64_t rows, uint64_t cols, uint64_t ld, const armx_config* cfg,
                   int cu_count, RowPlans* plans, bool allow_split) {
  RowPlans r;
  int st = make_plan(op, rows, cols, ld, cfg, cu_count, &r.main, allow_split);
  if (st != ARMX_OK) return st;
  const Plan& p = r.main;
  // Measured on MI355X (2^28 values): the second launch costs 8-16 us of
  // dispatch, ticket and latency, less than the extra round of the
  // fixed-order stream (2100 rows 101.4 -> 86.3 us, 2049 rows 95.6 -> 87.2)
  // but not always less than the free-order one's (4128 rows 86.3 -> 89.3),
  // so free order keeps its stream.
  if (allow_split && p.mode == 1 && op == kOpRowsFixed) {
    // the stream's wavefront count, and the rows of its last round
    const uint64_t T = uint64_t(p.grid) * uint64_t(p.waves);
    const uint64_t rounds = (rows + T - 1) / T;
    const uint64_t t = rows - (rounds - 1) * T;
    if (rounds >= 2 && 4 * t < 3 * T) {
      // two rounds: every row split in two aligned ranges, all in one launch,
      // which saves the second launch's dispatch and ticket (measured on
      // MI355X, 2^26 values: 1025 rows 29.6 -> 26.9 us, 1300 rows 32.0 ->
      // 27.6, 1500 rows 30.1 -> 27.3)
      // (only while the halves are all resident, one block per compute unit:
      // a grid larger than the unit count leaves some units two blocks)
      if (rounds == 2 && 2 * rows <= uint64_t(kMaxWaves) * uint64_t(cu_count) &&
          2 * rows <= kSplitMaxItems) {
        Plan h;
        if (make_plan(op, rows, cols, ld, cfg, cu_count, &h, true, true) == ARMX_OK &&
            h.mode == 3 && h.segs == 2) {
          r.main = h;
          *plans = r;
          return ARMX_OK;
        }
      }
      RowPlans s;
      s.tail_rows = t;
      if (make_plan(op, rows - t, cols, ld, cfg, cu_count, &s.main, true) == ARMX_OK &&
          make_plan(op, t, cols, ld, cfg, cu_count, &s.tail, true) == ARMX_OK &&
          s.main.mode == 1 && uint64_t(s.main.grid) * uint64_t(s.main.waves) == T &&
          s.tail.mode == 3) {
        s.main.stop_event = nullptr;   // the events bracket both launches
        s.tail.start_event = nullptr;
        r = s;
      }
    }
  }
  *plans = r;
  return ARMX_OK;
}

}  // namespace armx
