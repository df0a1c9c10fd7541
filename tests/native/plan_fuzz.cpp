// Host-only fuzz of the launch planner (plan.cpp): random operations, sizes
// and configurations; every accepted plan must satisfy the invariants the
// kernels rely on.  Built with AddressSanitizer and UBSan by
// tests/test_plan_fuzz.py.  Exit status 0 = all invariants held.
#include <cstdint>
#include <cstdio>
#include <random>

#include "plan.h"

using armx::Plan;

static int failures = 0;
#define EXPECT(cond, ...)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      ++failures;                                          \
      std::printf("violated: %s | ", #cond);               \
      std::printf(__VA_ARGS__);                            \
      std::printf("\n");                                   \
    }                                                      \
  } while (0)

static bool pow2(uint64_t v) { return v && !(v & (v - 1)); }
static uint64_t cdiv(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 200000;
  std::mt19937_64 rng(12345);
  auto pick_n = [&]() -> uint64_t {
    switch (rng() % 6) {
      case 0: return rng() % 64;
      case 1: return rng() % 100000;
      case 2: return uint64_t(1) << (rng() % 41);
      case 3: return (uint64_t(1) << (rng() % 41)) + (rng() % 1000) - 500;
      case 4: return rng() % (uint64_t(1) << 36);
      default: return rng();
    }
  };
  // fixed cases: the automatic row shapes
  {
    struct Case {
      int op;
      uint64_t rows, cols, ld;
      int mode, seg_log2, waves, r, remap;
    } cases[] = {
        {ARMX_OP_ROWS, 100000, 64, 64, 2, 3, 4, 4, 0},          // r: groups per step
        {ARMX_OP_ROWS_FIXED, 100000, 100, 104, 2, 4, 4, 8, 0},
        {ARMX_OP_ROWS, 100000, 8, 8, 2, 0, 4, 8, 1},
        {ARMX_OP_ROWS, 100000, 512, 512, 2, 6, 4, 4, 0},
        {ARMX_OP_ROWS, 300000, 1000, 1000, 1, 0, 8, 1, 1},
        {ARMX_OP_ROWS_FIXED, 300000, 1000, 1000, 1, 0, 4, 2, 1},   // 2 chunks ending inside one
        {ARMX_OP_ROWS_FIXED, 300000, 1024, 1024, 1, 0, 8, 2, 0},
        {ARMX_OP_ROWS_FIXED, 300000, 2048, 2048, 1, 0, 4, 4, 0},   // one group, blocks of 256
        {ARMX_OP_ROWS_FIXED, 77136, 3480, 3480, 1, 0, 4, 4, 1},    // 7 chunks
        {ARMX_OP_ROWS, 109297, 2456, 2456, 1, 0, 1, 3, 1},         // 5 chunks
        {ARMX_OP_ROWS, 65536, 4096, 4096, 1, 0, 1, 8, 0},
        {ARMX_OP_ROWS_FIXED, 65536, 4096, 4096, 1, 0, 1, 4, 0},
        {ARMX_OP_ROWS, 4096, 65536, 65536, 1, 0, 1, 8, 0},
        {ARMX_OP_ROWS, 57344, 4608, 4608, 1, 0, 1, 5, 0},        // 9 chunks: 5 + 4
        {ARMX_OP_ROWS, 16384, 16896, 16896, 1, 0, 1, 4, 0},      // 33 chunks: 8 would pad 7
        {ARMX_OP_ROWS, 67243, 3992, 3992, 1, 0, 1, 4, 1},        // 8 chunks ending inside one
        {ARMX_OP_ROWS, 26483, 10136, 10136, 1, 0, 1, 4, 1},      // 20 chunks: 3 chains of 8
        {ARMX_OP_ROWS, 24053, 11160, 11160, 1, 0, 1, 8, 1},      // 22 chunks: 8 pads 2
        {ARMX_OP_ROWS, 10528, 25496, 25496, 1, 0, 1, 8, 1},      // 50 chunks: 8 pads 6
        {ARMX_OP_ROWS, 4096, 65024, 65024, 1, 0, 1, 8, 0},       // 127 chunks: waste 1
        {ARMX_OP_ROWS_FIXED, 57344, 4608, 4608, 1, 0, 1, 2, 0},  // 9 chunks
        {ARMX_OP_ROWS_FIXED, 37449, 7168, 7168, 1, 0, 1, 2, 0},  // 14 chunks
        {ARMX_OP_ROWS_FIXED, 43690, 6144, 6144, 1, 0, 1, 4, 0},  // 12 chunks: tie
        {ARMX_OP_ROWS_FIXED, 4096, 66048, 66048, 1, 0, 1, 4, 0}, // 129: R 2 > 64 groups
    };
    for (const Case& k : cases) {
      Plan p;
      const int st = armx::make_plan(k.op, k.rows, k.cols, k.ld, nullptr, 256, &p);
      EXPECT(st == ARMX_OK, "fixed case status %d", st);
      EXPECT(p.mode == k.mode && p.seg_log2 == k.seg_log2 && p.waves == k.waves &&
                 (k.r < 0 || p.r == k.r) && p.xcd_remap == k.remap,
             "op %d %llux%llu ld %llu: mode %d seg %d waves %d r %d remap %d", k.op,
             (unsigned long long)k.rows, (unsigned long long)k.cols, (unsigned long long)k.ld,
             p.mode, p.seg_log2, p.waves, p.r, p.xcd_remap);
    }
  }
  // a grid cap is an upper bound on every plan, splits included
  {
    armx_config c{};
    c.grid_blocks = 10;
    for (int op : {ARMX_OP_ROWS, ARMX_OP_ROWS_FIXED}) {
      for (uint64_t rows : {uint64_t(900), uint64_t(1100), uint64_t(2049), uint64_t(3)}) {
        Plan p;
        const int st = armx::make_plan(op, rows, 20000, 20000, &c, 256, &p);
        EXPECT(st == ARMX_OK && p.grid <= 10, "grid cap: op %d rows %llu status %d grid %d",
               op, (unsigned long long)rows, st, p.grid);
        armx::RowPlans rp;
        EXPECT(armx::make_row_plans(op, rows, 20000, 20000, &c, 256, &rp) == ARMX_OK &&
                   rp.main.grid <= 10 && (!rp.tail_rows || rp.tail.grid <= 10),
               "grid cap (row plans): op %d rows %llu", op, (unsigned long long)rows);
      }
    }
  }
  // Flags each operation accepts, for the draws of valid configurations.
  auto valid_flags = [&](int op) -> unsigned {
    switch (op) {
      case ARMX_OP_SUM: {
        const unsigned k = unsigned(rng() % 4);
        if (k == 0) return ARMX_FLAG_MMA_LEVELS | unsigned(rng() % 2) * ARMX_FLAG_CACHED_LOADS;
        unsigned f = unsigned(rng() % 16);   // PLAIN, CACHED_LOADS, ONE_CHAIN, TWO_PASS
        if (!(f & ARMX_FLAG_PLAIN) && rng() % 2) f |= ARMX_FLAG_ALL_ONES;
        return f;
      }
      case ARMX_OP_FIXED:
        return unsigned(rng() % 2) * ARMX_FLAG_CACHED_LOADS |
               unsigned(rng() % 2) * ARMX_FLAG_TWO_PASS | unsigned(rng() % 2) * ARMX_FLAG_MMA_LEAVES;
      case ARMX_OP_ROWS: {
        const unsigned design = unsigned(rng() % 3);   // signed, plain, all ones
        return (design == 1 ? ARMX_FLAG_PLAIN : design == 2 ? ARMX_FLAG_ALL_ONES : 0u) |
               unsigned(rng() % 2) * ARMX_FLAG_CACHED_LOADS;
      }
      case ARMX_OP_ROWS_FIXED:
        return unsigned(rng() % 2) * ARMX_FLAG_CACHED_LOADS |
               unsigned(rng() % 2) * ARMX_FLAG_MMA_LEAVES;
      default:   // exact sum
        return unsigned(rng() % 2) * ARMX_FLAG_CACHED_LOADS |
               unsigned(rng() % 2) * ARMX_FLAG_INT_LIMBS;
    }
  };
  int accepted = 0;
  for (int it = 0; it < iters; ++it) {
    const int op = int(rng() % 6);  // 5 is not an operation
    armx_config c{};
    uint64_t n, cols, ld;
    const int cus = (rng() % 2) ? 256 : int(1 + rng() % 512);
    if (it % 2 == 0) {
      // anything, most of it invalid
      c.block_threads = (rng() % 4 == 0) ? 0 : int(rng() % 1200);
      if (rng() % 2) c.block_threads = 64 * int(1 + rng() % 16);
      c.chain_r = int(rng() % 10);
      c.grid_blocks = (rng() % 3 == 0) ? int(rng() % 5000) - 5 : 0;
      c.flags = unsigned(rng() % 256);
      n = pick_n();
      cols = pick_n() % (uint64_t(1) << 30);
      ld = (rng() % 2) ? cols : cols + (rng() % 64);
    } else {
      // valid configurations: automatic or power-of-two blocks, R 0..8,
      // flags the operation accepts; row counts near 1-4 times a row
      // stream's wavefront count, with long rows, half of the time
      c.block_threads = (rng() % 3 == 0) ? 0 : 64 << (rng() % 5);
      c.chain_r = int(rng() % 9);
      c.grid_blocks = (rng() % 3 == 0) ? int(1 + rng() % 3000) : 0;
      c.flags = valid_flags(op);
      if ((op == ARMX_OP_ROWS || op == ARMX_OP_ROWS_FIXED) && rng() % 2) {
        const uint64_t T = uint64_t(cus) * (1 + rng() % 16);
        n = T / 2 + rng() % (4 * T + 1);
        cols = 16384 + rng() % (uint64_t(1) << 20);
      } else {
        n = pick_n();
        cols = pick_n() % (uint64_t(1) << 24);
      }
      ld = (rng() % 2) ? cols : (cols + 7) / 8 * 8 + 8 * (rng() % 8);
    }
    Plan p;
    const int st = armx::make_plan(op, n, cols, ld, &c, cus, &p);
    if (op == 5) {
      EXPECT(st == ARMX_ERR_CONFIG, "op 5 accepted");
      continue;
    }
    EXPECT(st <= 0 && st >= ARMX_ERR_HIP, "status %d", st);
    if (st != ARMX_OK) continue;
    ++accepted;
    const uint64_t W = uint64_t(p.waves), R = uint64_t(p.r);
    EXPECT(W >= 1 && W <= 16 && R >= 1 && R <= 8, "W %llu R %llu", (unsigned long long)W,
           (unsigned long long)R);
    EXPECT(!(p.flags & ARMX_FLAG_MMA_LEAVES) || op == ARMX_OP_FIXED || op == ARMX_OP_ROWS_FIXED,
           "MMA leaves accepted for op %d", op);
    EXPECT(!(p.flags & ARMX_FLAG_INT_LIMBS) || op == ARMX_OP_EXACT,
           "integer limbs accepted for op %d", op);
    EXPECT(!(p.flags & ARMX_FLAG_ALL_ONES) ||
               ((op == ARMX_OP_SUM || op == ARMX_OP_ROWS) &&
                !(p.flags & (ARMX_FLAG_PLAIN | ARMX_FLAG_MMA_LEVELS))),
           "all-ones operand accepted for op %d flags 0x%x", op, p.flags);
    const bool levels = (p.flags & ARMX_FLAG_MMA_LEVELS) != 0;
    EXPECT(!levels || op == ARMX_OP_SUM, "levels flag accepted for op %d", op);
    if (levels) {
      EXPECT(!(p.flags & (ARMX_FLAG_PLAIN | ARMX_FLAG_TWO_PASS)), "levels flags");
      if (p.n == 0) continue;
      const uint64_t c1 = armx::level_count(p.n, R, 1), c2 = armx::level_count(c1, R, 2);
      if (c1 == 1) {
        EXPECT(p.ws_bytes == 0, "levels ws for one level");
      } else {
        EXPECT(p.partials_bytes >= 4 * c1 && p.partials_bytes % 256 == 0, "level-1 buffer");
        EXPECT(c2 == 1 ? p.aux_bytes == 0 : (p.aux_bytes >= 4 * c2 && p.aux_bytes % 256 == 0),
               "level-2 buffer");
        EXPECT(p.ws_bytes == armx::kCounterBytes + p.partials_bytes + p.aux_bytes, "levels ws");
      }
      // every level's chain count fits the level-k grid
      for (uint64_t c = c1; c > 1;) {
        c = armx::level_count(c, R, 2);
        EXPECT(cdiv(c, W) <= 0x7FFFFFFFull, "level grid");
      }
      continue;
    }
    if (op == ARMX_OP_EXACT) {
      EXPECT(!(p.flags & ~unsigned(ARMX_FLAG_CACHED_LOADS | ARMX_FLAG_INT_LIMBS)), "exact flags");
      EXPECT(!(p.flags & ARMX_FLAG_INT_LIMBS) || W * 64 <= armx::kExactLimbsMaxBlock,
             "limb form block %llu", (unsigned long long)(W * 64));
      if (p.n == 0) continue;
      EXPECT(p.grid >= 1 && uint64_t(p.grid) <= cdiv(cdiv(p.n, 512 * R), W), "exact grid");
      EXPECT(pow2(p.group) && cdiv(uint64_t(p.grid), p.group) <= armx::kMaxGroups, "groups");
      EXPECT(p.partials_bytes >= armx::kExactRecordBytes * uint64_t(p.grid) &&
             p.partials_bytes % 256 == 0, "exact records");
      EXPECT(p.ws_bytes >= armx::kCounterBytes + p.partials_bytes +
                              armx::kExactRecordBytes * armx::kMaxGroups, "exact ws");
      continue;
    }
    if (op == ARMX_OP_SUM || op == ARMX_OP_FIXED) {
      if (p.n == 0) continue;
      EXPECT(p.grid >= 1, "grid %d", p.grid);
      EXPECT(pow2(p.group), "group %u", p.group);
      EXPECT(cdiv(uint64_t(p.grid), p.group) <= armx::kMaxGroups, "groups");
      EXPECT(p.ws_bytes == armx::kCounterBytes + p.partials_bytes +
                             (4 * armx::kMaxGroups + 255) / 256 * 256,
             "ws layout");
      EXPECT(p.partials_bytes >= 4 * uint64_t(p.grid) && p.partials_bytes % 256 == 0, "partials");
    }
    if (op == ARMX_OP_SUM) {
      const uint64_t chains = cdiv(p.n, 512 * R);
      if (p.flags & ARMX_FLAG_ONE_CHAIN)
        EXPECT(uint64_t(p.grid) * W >= chains, "one chain: %d blocks x %llu waves < %llu chains",
               p.grid, (unsigned long long)W, (unsigned long long)chains);
      EXPECT(uint64_t(p.grid) <= cdiv(chains, W), "more blocks than chains need");
    }
    if (op == ARMX_OP_FIXED) {
      const uint64_t chunks = cdiv(p.n, 512);
      EXPECT(pow2(W), "fixed W %llu", (unsigned long long)W);
      EXPECT(p.grid <= armx::kFixedMaxBlocks, "fixed grid %d", p.grid);
      EXPECT((uint64_t(p.grid) * W << p.log2_chunks) >= chunks, "fixed coverage");
      EXPECT(((uint64_t(p.grid) - 1) * W << p.log2_chunks) < chunks, "fixed empty block");
      EXPECT(p.lds_bytes <= armx::kFixedLdsBytes, "lds %zu", p.lds_bytes);
      EXPECT(p.lds_bytes == W * p.slots_per_wave * sizeof(float), "lds size");
      EXPECT(p.slots_per_wave % 64 == 0, "slots %u", p.slots_per_wave);
      const uint64_t per_node = pow2(R) ? R : 1;
      EXPECT(uint64_t(p.slots_per_wave) >= cdiv(uint64_t(1) << p.log2_chunks, per_node),
             "slots too few");
    }
    if (op == ARMX_OP_ROWS || op == ARMX_OP_ROWS_FIXED) {
      // the call's plans: a stream of full rounds plus a split tail, or one plan
      armx::RowPlans rp;
      EXPECT(armx::make_row_plans(op, n, cols, ld, &c, cus, &rp) == ARMX_OK, "row plans");
      if (rp.tail_rows) {
        const uint64_t T = uint64_t(rp.main.grid) * uint64_t(rp.main.waves);
        EXPECT(op == ARMX_OP_ROWS_FIXED, "tail for free-order rows");
        EXPECT(rp.main.rows + rp.tail_rows == n, "tail covers the last rows");
        EXPECT(rp.main.mode == 1 && rp.main.rows % T == 0 && rp.main.rows >= T,
               "head of full rounds");
        EXPECT(rp.tail.mode == 3 && 4 * rp.tail_rows < 3 * T, "split tail");
        EXPECT(rp.ws_bytes() == rp.tail.ws_bytes && rp.main.ws_bytes == 0, "tail workspace");
        EXPECT(rp.main.stop_event == nullptr && rp.tail.start_event == nullptr, "tail events");
      } else if (op == ARMX_OP_ROWS_FIXED && p.mode == 1 && rp.main.mode == 3) {
        // two rounds, the second poorly filled: every row in two ranges
        const uint64_t T = uint64_t(p.grid) * uint64_t(p.waves);
        EXPECT(rp.main.segs == 2 && n > T && n <= 2 * T && 4 * (n - T) < 3 * T &&
                   2 * n <= uint64_t(armx::kMaxWaves) * uint64_t(cus),
               "rows in halves");
        EXPECT(rp.main.rows == n && rp.ws_bytes() == rp.main.ws_bytes && rp.main.ws_bytes > 0,
               "halves workspace");
      } else {
        EXPECT(rp.main.mode == p.mode && rp.main.grid == p.grid && rp.ws_bytes() == p.ws_bytes,
               "one row plan");
      }
      EXPECT(c.grid_blocks <= 0 ||
                 (rp.main.grid <= c.grid_blocks && (!rp.tail_rows || rp.tail.grid <= c.grid_blocks)),
             "row plans grid cap");
      armx::RowPlans rq;
      EXPECT(armx::make_row_plans(op, n, cols, ld, &c, cus, &rq, false) != ARMX_OK ||
                 rq.tail_rows == 0,
             "tail without a workspace");
      EXPECT(p.ld >= p.n, "ld");
      // only a split (mode 3) uses a workspace: the counter region and one
      // partial per wavefront
      if (p.mode == 3) {
        EXPECT(p.ws_bytes == armx::kCounterBytes + (4 * p.rows * p.segs + 255) / 256 * 256,
               "split workspace %zu", p.ws_bytes);
        EXPECT(p.segs >= 2 && p.segs <= armx::kSplitMaxSegs, "segs %u", p.segs);
        EXPECT(uint64_t(p.grid) == cdiv(p.rows * p.segs, W), "split grid %d", p.grid);
        EXPECT(uint64_t(p.grid) <= armx::kSplitMaxBlocks, "split grid %d", p.grid);
        EXPECT(p.rows * p.segs <= armx::kSplitMaxItems, "split parts %llu",
               (unsigned long long)(p.rows * p.segs));
        EXPECT(c.grid_blocks <= 0 || p.grid <= c.grid_blocks, "split grid cap");
        EXPECT(p.n > 512, "split of short rows");
        // the same call without a workspace plans no split (fixed-order rows
        // too long for one block's node logs are then refused)
        Plan q;
        const int sq = armx::make_plan(op, n, cols, ld, &c, cus, &q, false);
        EXPECT((sq == ARMX_OK && q.mode != 3 && q.ws_bytes == 0) ||
                   (sq == ARMX_ERR_SHAPE && op == ARMX_OP_ROWS_FIXED),
               "split without a workspace: status %d", sq);
      } else {
        EXPECT(p.ws_bytes == 0, "rows workspace");
      }
      if (p.rows == 0 || p.n == 0) continue;
      EXPECT(p.grid >= 1 && uint64_t(p.grid) <= (uint64_t(1) << 20), "rows grid %d", p.grid);
      if (p.rows > 1) EXPECT(p.ld % 8 == 0, "pitch");
      // XCD-contiguous block order for rows that share lines, except in the
      // staged short-row kernel, whose blocks take whole chunks of rows
      const bool staged = p.mode == 2 && p.seg_log2 >= armx::kShortStagedMinLog2;
      EXPECT(p.xcd_remap == (p.rows > 1 && p.ld % 64 != 0 && !staged ? 1 : 0), "remap %d",
             p.xcd_remap);
      // rows of at most one chunk take the segmented kernel, with the
      // smallest power-of-two lane count that holds a row
      EXPECT((p.mode == 2) == (p.n <= 512), "short-row mode %d for %llu columns", p.mode,
             (unsigned long long)p.n);
      if (p.mode == 2) {
        const uint64_t lanes = cdiv(p.n, 8), P = uint64_t(1) << p.seg_log2;
        EXPECT(p.seg_log2 >= 0 && p.seg_log2 <= 6, "seg_log2 %d", p.seg_log2);
        EXPECT(P >= lanes && (P == 1 || P / 2 < lanes), "lanes per row");
        // 4 groups per step for staged rows at a whole-line pitch, else 8
        EXPECT(p.r == (p.seg_log2 >= armx::kShortStagedMinLog2 && (p.rows == 1 || p.ld % 64 == 0)
                           ? 4 : 8),
               "short-row groups %d", p.r);
        const uint64_t rps = (64 / P) * uint64_t(p.r);
        const uint64_t steps = cdiv(p.rows, rps);
        EXPECT(c.grid_blocks <= 0 || p.grid <= c.grid_blocks, "short-row grid cap");
        if (p.seg_log2 >= armx::kShortStagedMinLog2) {
          // a chunk (a block's share) is at least one step
          EXPECT(uint64_t(p.grid) <= steps, "short-row grid %d", p.grid);
          // chunks of whole steps that fit the LDS, and no more blocks than chunks
          EXPECT(p.chunk_rows >= rps && p.chunk_rows % rps == 0 &&
                     p.chunk_rows <= armx::kShortChunkRows,
                 "short-row chunk %llu", (unsigned long long)p.chunk_rows);
          EXPECT(p.lds_bytes == p.chunk_rows * sizeof(float), "short-row lds");
          const uint64_t body = p.rows - (p.n % 8 ? 1 : 0);
          EXPECT(uint64_t(p.grid) <= (body ? cdiv(body, p.chunk_rows) : 1), "short-row chunks");
        } else {
          EXPECT(uint64_t(p.grid) <= cdiv(steps, W), "short-row grid %d", p.grid);
          EXPECT(p.chunk_rows == 0 && p.lds_bytes == 0, "short-row lds");
        }
        EXPECT(!(p.flags & ARMX_FLAG_MMA_LEAVES) || W * 64 <= armx::kShortMmaMaxBlock,
               "MFMA-leaf short-row block %llu", (unsigned long long)(W * 64));
      }
    }
    if (op == ARMX_OP_ROWS && p.mode == 3)
      EXPECT(p.segs <= cdiv(p.n, 512 * R), "more segments than chains");
    if (op == ARMX_OP_ROWS_FIXED && p.mode == 3) {
      // aligned power-of-two ranges that cover the row, none empty
      const uint64_t chunks = cdiv(p.n, 512), span = uint64_t(1) << p.log2_chunks;
      EXPECT(uint64_t(p.segs) * span >= chunks && uint64_t(p.segs - 1) * span < chunks,
             "split coverage");
      EXPECT(p.segs <= armx::kSplitMaxSegs, "segs %u", p.segs);
      EXPECT(p.lds_bytes + armx::kSplitMaxItems * sizeof(float) <= armx::kFixedLdsBytes,
             "split lds");
      EXPECT(p.lds_bytes == W * p.slots_per_wave * sizeof(float), "split lds size");
      const uint64_t per_node = pow2(R) ? R : 1;
      EXPECT(p.slots_per_wave % 64 == 0 && uint64_t(p.slots_per_wave) >= cdiv(span, per_node),
             "split slots");
    }
    if (op == ARMX_OP_ROWS_FIXED) {
      EXPECT(pow2(W) || p.mode == 3, "rows fixed W");
      if (p.mode == 1) {
        EXPECT(pow2(R) && cdiv(p.n, 512 * R) <= 64, "flat shape");
      } else if (p.mode == 0) {
        EXPECT((W << p.log2_chunks) >= cdiv(p.n, 512), "rows fixed coverage");
        EXPECT(p.lds_bytes <= armx::kFixedLdsBytes, "rows fixed lds");
        EXPECT(p.lds_bytes == W * p.slots_per_wave * sizeof(float), "rows fixed lds size");
      }
    }
  }
  std::printf("plans accepted %d of %d, violations %d\n", accepted, iters, failures);
  return failures ? 1 : 0;
}
