// Launch planning shared by the C entry points and the kernel launchers.
// Plain C++: no HIP types, so argument checking and grid sizing can be
// exercised without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "armx.h"

namespace armx {

// One wavefront load: 64 lanes x 16 bytes = 512 binary16 values.  It is also
// one B operand of v_mfma_f32_16x16x32_f16 (32 x 16 values).
constexpr uint64_t kChunk = 512;
// Leaf tile of the fixed-order tree (a complete depth-8 subtree).
constexpr uint64_t kTile = 256;
constexpr int kMaxR = 8;
constexpr int kMaxWaves = 16;
// Per-operation defaults (block threads, chain length R) and the number of
// 16-byte loads per lane an automatic persistent grid keeps in flight per
// compute unit: an HBM stream is latency-bound unless enough bytes are in
// flight, and measured on MI355X fewer, deeper streams do best, so the grid
// holds about loads_per_cu / R wavefronts per compute unit (and at least one
// block per compute unit).
struct OpDefaults {
  int block;
  int r;
  int loads_per_cu;
};
constexpr OpDefaults kSumDefaults{128, 8, 16};
constexpr OpDefaults kFixedDefaults{128, 8, 16};
constexpr OpDefaults kRowsDefaults{64, 8, 16};
// fixed-order rows: measured on MI355X, R = 4 (4 wavefronts per CU) hides the
// per-group tree work best on 4096 x 65536 (76.9 us against 82.6 us at R = 8)
constexpr OpDefaults kRowsFixedDefaults{64, 4, 16};
// The MMA-levels form: its level-1 chains end in a longer dependent MFMA
// sequence, and measured on MI355X more wavefronts per compute unit (about 8
// at R = 8) hide it best.
constexpr OpDefaults kLevelsDefaults{256, 8, 64};
constexpr OpDefaults kExactDefaults{128, 8, 16};
// Exact sum: each block publishes a 32-byte record (two 64-bit limbs, flags).
constexpr size_t kExactRecordBytes = 32;
// Largest block of the exact sum's integer-limb form (ARMX_FLAG_INT_LIMBS):
// its digit words need more registers than a 1024-thread block leaves a lane;
// a larger requested block is lowered to this.
constexpr int kExactLimbsMaxBlock = 512;
// Its defaults: about 14 vector instructions per value make it bound by the
// vector ALUs, which want every SIMD busy -- measured on MI355X at 2^28 values
// (us, events around 50 calls, two copies in turn): blocks of 512 at R = 4
// (8 wavefronts per CU) 111.9, R = 2 117.7, R = 8 137.9; blocks of 256 at
// R = 4 114.1, R = 8 116.7; blocks of 128 at R = 8 (2 per CU) 212.2.
constexpr OpDefaults kExactLimbsDefaults{512, 4, 16};
// The fixed-order final combine handles at most this many block results.
constexpr int kFixedMaxBlocks = 4096;
// Largest fixed-order per-wave chunk count is 2^kFixedMaxLog2Chunks.
constexpr int kFixedMaxLog2Chunks = 24;
// Fixed order keeps each wavefront's node log in LDS: at most this much per block.
constexpr size_t kFixedLdsBytes = 64 * 1024;
// Workspace: the completion counters (one top counter and at most
// kMaxGroups group counters) sit in the first kCounterBytes, each counter at
// the start of its own 256-byte stretch (kCounterStride 32-bit words): device
// atomics on counters that share those bytes are served one after another
// (measured on MI355X, 2^28 values, one chain per wavefront, 64-thread blocks
// at R = 5: 1105 us with the 64 counters packed in 256 bytes, 187 us spread,
// 99 us spread with up to 255 groups).
constexpr unsigned kCounterStride = 64;
// A single ticket group whose blocks may split their counting (short
// streams) counts them in runs of this many blocks, one counter per run.
constexpr unsigned kSplitCountRun = 16;
constexpr unsigned kMaxGroups = 255;
constexpr size_t kCounterBytes = size_t(1 + kMaxGroups) * kCounterStride * sizeof(unsigned);
static_assert(kCounterBytes == ARMX_COUNTER_BYTES, "the header's counter region size");
constexpr uint64_t kMaxN = uint64_t(1) << 40;
// The static scratch array of reduce_sum_noalloc (one per device): calls
// whose plan needs a larger workspace are refused.
constexpr size_t kScratchBytes = size_t(1) << 20;

enum Op {
  kOpSum = ARMX_OP_SUM,
  kOpRows = ARMX_OP_ROWS,
  kOpFixed = ARMX_OP_FIXED,
  kOpRowsFixed = ARMX_OP_ROWS_FIXED,
  kOpExact = ARMX_OP_EXACT
};

struct Plan {
  int op = 0;
  int waves = 0;            // wavefronts per block (W)
  int r = 0;                // loads per wavefront per step (R)
  int grid = 0;             // blocks launched
  unsigned flags = 0;
  int log2_chunks = 0;      // fixed order: 2^log2_chunks chunks per wavefront
  int mode = 0;             // rows: 1 = one wavefront per row, 0 = one block per row;
                            // fixed-order rows: 1 = flat (cross-row stream), 0 = general;
                            // both: 2 = rows of at most one chunk, segmented lanes;
                            // 3 = each row split over `segs` wavefronts of several
                            // blocks, combined by the last block (a workspace)
  int seg_log2 = 0;         // mode 2: log2 of the lanes per row (a power of two)
  unsigned segs = 0;        // mode 3: wavefronts (row segments) per row
  int xcd_remap = 0;        // rows: give each XCD a contiguous range of block ids
  unsigned slots_per_wave = 0;  // fixed order: LDS floats of each wavefront's node log
  size_t lds_bytes = 0;     // dynamic LDS per block
  uint64_t n = 0;           // elements (sum / fixed); columns (rows)
  uint64_t rows = 0;
  uint64_t ld = 0;
  uint64_t chunk_rows = 0;  // mode 2: rows a block reduces into LDS before writing them
  size_t ws_bytes = 0;      // workspace the launch needs
  size_t partials_bytes = 0;  // block-result region of the workspace (MMA levels:
                              // the first level buffer)
  size_t aux_bytes = 0;       // MMA levels: the second level buffer
  unsigned group = 1;       // blocks per completion group (a power of two)
  void* start_event = nullptr;  // hipEvent_t stamped around the main kernel
  void* stop_event = nullptr;
};

// Request pacing (device_common.hpp, pace_pause): streams of at least
// kPaceLongChains chains (or groups) per wavefront take the long pause,
// those of at least kPaceShortChains the short one.
constexpr uint64_t kPaceLongChains = 64;
constexpr uint64_t kPaceShortChains = 8;

// Rows of at most one chunk (mode 2): each wavefront takes G groups of
// 64 / 2^S rows per step (S = seg_log2, G = the plan's r), one 16-byte load
// per lane each, and the persistent grid holds kShortWavesPerCu wavefronts
// per compute unit (measured on MI355X at 2^28 values: 4 beat 2 and 8 for 64
// to 512 columns, best as one block of 4 wavefronts).
//  * Rows of more than 32 values (S >= kShortStagedMinLog2) are cut into
//    chunks of at most kShortChunkRows consecutive rows; a block reduces a
//    chunk into LDS and writes the chunk's sums out together (4194304 rows of
//    64 values: 87.4 -> 80.6 us against every wavefront storing its sums step
//    by step; 128 to 512 values 1-6 us faster).  G = 4 when the row pitch is
//    a whole number of 128-byte lines, else 8 (2581110 rows of 100 values at
//    a pitch of 104: 83.3 us at G = 4 against 81.4 at G = 8, and 91.0 against
//    81.1 with MFMA leaves; at a pitch of 64, 80.6 against 83.4).
//  * Narrower rows write as they go, G = 8: their sums are 1/8 to 1/2 of the
//    input bytes, more than a chunk of LDS holds for the grid to stream on
//    while it is written out (33554432 rows of 8 values: 104.7 us writing as
//    they go, 116-125 us through LDS).
constexpr int kShortWavesPerCu = 4;
constexpr int kShortBlock = 256;   // automatic block size for such rows
constexpr int kShortStagedMinLog2 = 3;
constexpr uint64_t kShortChunkRows = 16384;   // 64 KiB of LDS
// Largest block of the MFMA-leaf kernel for such rows: its two reduction
// paths need more than the 128 registers a 1024-thread block leaves a lane
// (a larger requested block is lowered to this; a row's result never depends
// on the block).
constexpr int kShortMmaMaxBlock = 256;

// Rows too few to give the persistent grid's wavefronts one row each (mode
// 3): every row is split over several wavefronts in different blocks, each
// publishing a part; one completion counter (the grid is at most
// kSplitMaxBlocks blocks, within what the flat sums' single-level ticket
// takes) lets the last block stage all rows x S parts (at most
// kSplitMaxItems) in LDS and write every row's tree over its parts, at most
// kSplitMaxSegs of them (8 per lane).  Fixed order cuts a row into aligned
// power-of-two chunk ranges.  An automatic block size is the part count over
// the compute-unit count, rounded up (not a power of two), so no compute unit
// gets a second block.  A split pays for its completion ticket (a few
// microseconds) only when a wavefront's share of a row without it is large:
// at least kSplitMinShare values (64 KiB); no segment is made smaller than
// kSplitMinSegment values.
// Free-order row streams (one wavefront per row) of rows of at least
// kRowsLongMinCols values, in blocks of at most kRowsStreamMaxBlock threads,
// run as a kernel of their own, compiled for such blocks (more registers per
// wavefront than a kernel that may run 1024-thread blocks).
constexpr int kRowsStreamMaxBlock = 512;
constexpr uint64_t kRowsLongMinCols = 32768;
// Row streams read rows of fewer values than this through range-checked
// buffer loads (32-bit byte offsets and record counts).
constexpr uint64_t kRowsRangeMaxCols = uint64_t(1) << 29;

constexpr uint64_t kSplitMaxBlocks = 512;
constexpr uint64_t kSplitMaxItems = 8192;
static_assert(kSplitMaxItems == kSplitMaxBlocks * kMaxWaves, "a split grid's parts fit the stage");
constexpr uint64_t kSplitMaxSegs = 512;
constexpr uint64_t kSplitMinShare = 32768;
constexpr uint64_t kSplitMinSegment = 8192;

// MMA levels (ARMX_FLAG_MMA_LEVELS): the number of fp32 values level `level`
// produces from `count` inputs -- one per chain of R x 512 binary16 values at
// level 1, one per chain of R x 256 fp32 values above.
inline uint64_t level_count(uint64_t count, uint64_t r, int level) {
  const uint64_t per_chain = r * (level == 1 ? kChunk : 256);
  return (count + per_chain - 1) / per_chain;
}

// Resolves and checks a configuration for `op`.  `cu_count` is the number of
// compute units of the target device.  `allow_split` lets the row entry
// points plan mode 3 (which needs a workspace).  Returns ARMX_OK or a
// negative status; pointers are not examined here.
// `split_in_halves` (fixed-order rows, with allow_split) plans the split with
// two aligned ranges per row whatever the row count.
int make_plan(int op, uint64_t n_or_rows, uint64_t cols, uint64_t ld,
              const armx_config* cfg, int cu_count, Plan* plan, bool allow_split = true,
              bool split_in_halves = false);

// The launches of one row call: the main plan and, when a fixed-order row
// stream's last round of rows would be poorly filled (under three quarters),
// either (two rounds) one split launch with every row in two aligned ranges,
// or a second launch for that round's `tail_rows` rows -- the last rows of
// the matrix -- split over the whole device, so the stream runs full rounds
// only.  Needs the split's workspace; without one (allow_split false) there
// is neither.
struct RowPlans {
  Plan main;
  Plan tail;
  uint64_t tail_rows = 0;
  size_t ws_bytes() const { return tail_rows ? tail.ws_bytes : main.ws_bytes; }
};

int make_row_plans(int op, uint64_t rows, uint64_t cols, uint64_t ld, const armx_config* cfg,
                   int cu_count, RowPlans* plans, bool allow_split = true);

}  // namespace armx
