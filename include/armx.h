/*
 * armx.h -- fp16 sum-reduction on AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operation is the arithmetic reduction (sum) of n numbers, computed as
 * chained matrix-multiply-accumulates whose other operand is all ones, with
 * 32-bit float sub-results per chain and a 32-bit float final result:
 *   "GPU Tensor Cores for fast Arithmetic Reductions" (arXiv 2001.05585),
 *   Abstract.
 * The fixed-order entry point follows the balanced-tree reduction order used
 * to make results bitwise reproducible in
 *   "Taming Bitwise Behavior in GPU Kernels with Tensor Core: Black-Box
 *   Reconstruction, Compiler Enforcement, and Static Verification"
 *   (arXiv 2609.11356), Abstract.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Inputs are IEEE binary16 ("fp16") values, little-endian, in device
 *   memory.  Outputs are IEEE binary32 values in device memory.
 * - All pointers except `cfg` are DEVICE pointers on the current HIP device.
 *   `cfg` is a HOST pointer and may be NULL (all defaults).
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *   call only enqueues work on `stream` and returns; results are ready when
 *   the stream reaches that point.  Nothing is copied to the host and the
 *   host is never synchronised.
 * - The caller owns every buffer.  The library allocates no memory and keeps
 *   no state between calls other than a per-device cache of the compute-unit
 *   count.  Outputs and the workspace must not overlap the input or each
 *   other (the kernels read x while results are written).
 * - Errors are returned as a negative armx_status before anything is
 *   enqueued; the library never aborts, and prints nothing unless the
 *   environment variable ARMX_LOG is set, in which case every accepted call
 *   writes one line with its launch plan (grid, block size, R, workspace) to
 *   stderr.  A failure reported by the HIP runtime while enqueueing returns
 *   ARMX_ERR_HIP.
 * - Workspace: `ws` points to at least armx_workspace_bytes(...) bytes,
 *   256-byte aligned.  Its first ARMX_COUNTER_BYTES bytes hold the
 *   completion counters, which MUST be zero before the first call that uses
 *   the buffer; every call leaves them zero again when it completes, so
 *   zero-filling a workspace once after allocating it is enough.  Calls that may run at the same time
 *   (different streams) need different workspaces.  When the required size
 *   is 0, ws may be NULL.
 * - Non-finite inputs follow IEEE addition: any NaN, or +Inf together with
 *   -Inf, gives NaN; otherwise an infinity gives that infinity.
 * - Inputs that are binary16 subnormals are converted exactly (never
 *   flushed to zero).
 */
#ifndef ARMX_H
#define ARMX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Size of the counter region at the start of every non-empty workspace: a
 * top counter and up to 255 group counters, each at the start of its own
 * 256 bytes (device atomics on counters that share 256 bytes are served one
 * at a time). */
#define ARMX_COUNTER_BYTES 65536u

typedef enum armx_status {
  ARMX_OK = 0,
  ARMX_ERR_NULL = -1,      /* a required pointer is NULL                         */
  ARMX_ERR_ALIGN = -2,     /* x not 16-byte aligned, ws not 256-byte aligned, or */
                           /* a row pitch that is not a multiple of 8 elements   */
  ARMX_ERR_CONFIG = -3,    /* block size, chain length, grid or flags invalid    */
  ARMX_ERR_WORKSPACE = -4, /* ws_bytes smaller than armx_workspace_bytes()       */
  ARMX_ERR_SHAPE = -5,     /* ld < cols, or a size too large to index            */
  ARMX_ERR_HIP = -6        /* the HIP runtime reported an error                  */
} armx_status;

/* Flags for armx_config.flags. */
#define ARMX_FLAG_PLAIN 0x1u       /* reduce_sum / reduce_rows: the MFMA-free   */
                                   /* comparison design -- each lane converts  */
                                   /* its fp16 values and adds them in fp32,   */
                                   /* then cross-lane and block combines       */
#define ARMX_FLAG_CACHED_LOADS 0x2u /* read the input with ordinary loads;     */
                                    /* by default it is streamed with          */
                                    /* non-temporal loads                      */
#define ARMX_FLAG_ONE_CHAIN 0x4u   /* reduce_sum: every wavefront runs exactly */
                                   /* one chain of R tiles, so the grid is     */
                                   /* ceil(n / (512 R W)) blocks of W waves;   */
                                   /* without it a persistent grid loops       */
#define ARMX_FLAG_TWO_PASS 0x8u    /* reduce_sum / fixed order: a second launch */
                                   /* combines the block results instead of    */
                                   /* the last block to finish                 */
#define ARMX_FLAG_MMA_LEVELS 0x10u /* reduce_sum: the recursive all-MMA form   */
                                   /* (see reduce_sum); not with PLAIN or      */
                                   /* TWO_PASS                                 */
#define ARMX_FLAG_MMA_LEAVES 0x20u /* the two fixed-order entry points: the    */
                                   /* order whose leaves are MFMAs (see        */
                                   /* reduce_sum_fixed_order)                  */
#define ARMX_FLAG_INT_LIMBS 0x80u  /* reduce_sum_exact: the sums as integer    */
                                   /* MFMAs over 8-bit limbs (see              */
                                   /* reduce_sum_exact)                        */
#define ARMX_FLAG_ALL_ONES 0x40u   /* reduce_sum / reduce_rows: the MFMA       */
                                   /* design with the literal all-ones operand */
                                   /* (see reduce_sum); not with PLAIN or      */
                                   /* MMA_LEVELS                               */

typedef struct armx_config {
  int block_threads; /* 0 = default; else 64..1024, a multiple of 64.         */
                     /* reduce_sum_fixed_order needs a power of two.          */
  int chain_r;       /* 0 = default; else 1..8.  The number of 16-byte loads  */
                     /* (and, for the MFMA design, chained MFMAs) per         */
                     /* wavefront per loop step.                              */
  int grid_blocks;   /* 0 = automatic; else an upper bound on the grid.       */
  unsigned flags;    /* ARMX_FLAG_* bits.                                     */
  void* start_event; /* optional hipEvent_t (NULL = none): stamped by the     */
  void* stop_event;  /* dispatch packet of the main kernel when it starts and */
                     /* when it completes (hipExtLaunchKernel), so          */
                     /* hipEventElapsedTime gives that kernel's own duration */
} armx_config;
/* Defaults (block_threads, chain_r), measured on MI355X:
 *   reduce_sum 128, 8; reduce_sum_fixed_order 128, 8; reduce_rows 64, 8;
 *   reduce_rows_fixed_order 64, 4; reduce_sum with ARMX_FLAG_MMA_LEVELS
 *   256, 8; reduce_sum_exact 128, 8 (with ARMX_FLAG_INT_LIMBS 512, 4, and
 *   larger blocks lowered to 512).
 * Automatic persistent grids hold about 16 / R wavefronts per compute unit
 * (2 at the default R: fewer, deeper load streams reach more HBM bandwidth;
 * 64 / R for the MMA-levels form), and at least one block per compute
 * unit.  Inputs too small to feed that grid use about sqrt(n) / R
 * wavefronts instead (the flat sums: fewer blocks finish sooner when each
 * has little to stream).
 * The row entry points pick their defaults by row length: rows of at most
 * 512 values take the segmented kernel (block 256, 4 wavefronts per compute
 * unit, 4 or 8 loads per step -- 4 for rows of more than 32 values at a pitch
 * of whole 128-byte lines -- which armx_launch_plan reports as chain_r;
 * chain_r has no effect there; rows of more than 32 values use up to 64 KiB
 * of LDS per block to hold a chunk of row sums); rows of 513 to 3584 values
 * (2 to 7 chunks of 512): free order R = 1 in blocks of 512 threads, and,
 * when there are at least 64 rows per compute unit, R = 2 for rows of 4, 6
 * or 7 chunks and R = 3 in blocks of 64 for rows of 5; fixed order R = 1 in
 * blocks of 256, a row of exactly 2 or 4 chunks one group (R = 2 in blocks
 * of 512, R = 4 in blocks of 512, or of 256 with at least 64 rows per
 * compute unit), and with at least 64 rows per compute unit R = 2 in blocks
 * of 256 for other rows of 2, 4 or 6 chunks and R = 4 in blocks of 256 for
 * rows of 7; longer
 * rows, with the default block size: fixed order the R of 2 and 4 that
 * leaves a row's last group of R chunks the least padding; free order, rows
 * of 8 to 13 chunks the R of 8, 5 and 4 that pads the last chain least (rows
 * of 8 chunks that end inside the last: R = 4), rows of 14 chunks or more
 * R = 8 when that pads the last chain by at most a fifth of the row (below
 * 22 chunks: by at most one chunk), else R = 4.  An explicit
 * block_threads or chain_r overrides its part, except that rows of at most
 * 512 values with ARMX_FLAG_MMA_LEAVES run blocks of at most 256 threads (a
 * larger block_threads is lowered; no row's result depends on it). */

/*
 * reduce_sum -- out[0] = sum of x[0..n), free summation order.
 *
 *   "GPU Tensor Cores for fast Arithmetic Reductions", Abstract: the sum of n
 *   numbers encoded as chained m x m matrix-multiply-accumulates, each chain
 *   of R kept as a 32-bit float, then all chain results reduced to one
 *   32-bit float.
 *
 * x        device, n binary16 values, contiguous, 16-byte aligned (any
 *          alignment when n == 0; may be NULL when n == 0).
 * n        element count, 0 .. 2^40.
 * out      device, 1 binary32; n == 0 writes +0.0.
 * ws       device workspace (see conventions), ws_bytes its size.
 * cfg      host, may be NULL.  ARMX_FLAG_PLAIN selects the MFMA-free design,
 *          ARMX_FLAG_ALL_ONES the all-ones operand.
 *
 * Each wavefront multiplies a constant 16x32 fp16 matrix of ones by 32x16
 * tiles of x (one 16-byte load per lane) with v_mfma_f32_16x16x32_f16,
 * chaining R of them into fp32 accumulators.  By default the ones matrix has
 * its lower 8 rows negated: D's upper rows accumulate the 16 column sums and
 * its lower rows their negations, each element on its own, and the result is
 * half the difference of the two totals.  The MFMA's accumulation on gfx950
 * cuts some low bits toward minus infinity, which makes an all-ones sum lean
 * low on data of wide dynamic range (measured: -10 on a sum of 2^30 values
 * whose exact value is 9797); the negated sums lean the other way by the
 * same amount in distribution, so the difference cancels the lean.  It costs
 * no instruction per load.  ARMX_FLAG_ALL_ONES selects the literal all-ones
 * operand (every output row a column sum; the total read from one row).  The
 * order of additions depends on the configuration (not on timing): two calls
 * with the same n, configuration and device give the same bits.
 *
 * With ARMX_FLAG_MMA_LEVELS the sum is computed in the recursive form whose
 * level count the same Abstract's running-time model T(n) = 5 log_{m^2}(n)
 * counts: level 1 reduces every chain of R x 512 values to one fp32 with
 * MFMAs only (the tiles as the A operand against ones give 16 row sums; four
 * v_mfma_f32_16x16x4_f32 against ones add those), and each further level
 * reduces chains of R x 256 fp32 values of the level below the same way,
 * one launch per level, until one value is left.  Its result depends on n
 * and R only (not on block size or grid).  The workspace holds the level
 * buffers: about 4 * ceil(n / (512 R)) bytes plus the counter region (0
 * bytes when n <= 512 R); the counter region is left untouched.  start_event
 * is stamped by the first level's launch and stop_event by the last.
 * Returns ARMX_OK or ARMX_ERR_{NULL,ALIGN,CONFIG,WORKSPACE,SHAPE,HIP}.
 */
int reduce_sum(const void* x, size_t n, float* out, void* ws, size_t ws_bytes,
               const armx_config* cfg, void* stream);

/*
 * reduce_rows -- out[r] = sum over c < cols of x[r * ld + c], r < rows.
 *
 *   A row-segmented form of the same reduction (many independent sums of the
 *   Abstract of "GPU Tensor Cores for fast Arithmetic Reductions"), free
 *   summation order inside each row.
 *
 * x        device, row-major binary16, row r starts at element r * ld;
 *          16-byte aligned; ld must be a multiple of 8 when rows > 1.
 * rows     number of rows (0 writes nothing).
 * cols     elements summed per row (0 writes +0.0 to every row).
 * ld       row pitch in elements, ld >= cols.
 * out      device, rows binary32 values.
 * ws       device workspace (see conventions), or NULL.  When the rows are
 *          too few for the device (under three quarters of the wavefronts
 *          of its persistent grid) and long, or more but with a last round
 *          of rows under 90% full (up to four rounds), armx_workspace_bytes
 *          is non-zero and, with a workspace, every row is split over
 *          several wavefronts in different blocks whose partial sums the
 *          last block to finish combines in a fixed order; with ws NULL
 *          those rows are summed as without a split (slower, and in another
 *          order).  Otherwise ws is not used.
 * cfg      host, may be NULL.  ARMX_FLAG_PLAIN selects the MFMA-free design,
 *          ARMX_FLAG_ALL_ONES the all-ones operand (see reduce_sum).
 * Returns ARMX_OK or ARMX_ERR_{NULL,ALIGN,CONFIG,WORKSPACE,SHAPE,HIP}.
 *
 * Rows of at most 512 values are summed by lanes (each row on a
 * power-of-two group of lanes, several rows per wavefront load) in the
 * balanced-tree order of reduce_rows_fixed_order, with or without
 * ARMX_FLAG_PLAIN: an all-ones MFMA would add values of lanes 16 apart,
 * which there belong to different rows.  Reads may cover the pitch padding
 * of a row (never past the last row's cols values); its contents never
 * reach the result.
 */
int reduce_rows(const void* x, size_t rows, size_t cols, size_t ld, float* out,
                void* ws, size_t ws_bytes, const armx_config* cfg, void* stream);

/*
 * reduce_sum_fixed_order -- out[0] = sum of x[0..n) in one prescribed order.
 *
 *   "Taming Bitwise Behavior in GPU Kernels with Tensor Core", Abstract:
 *   reduction order is the main cause of bit-level differences, and a
 *   balanced-tree order makes a reduction reproducible.
 *
 * The result is the root of the balanced binary tree over x[0..n) padded
 * with -0.0 to the next power of two, every node the binary32
 * round-to-nearest-even sum of its two children (leaves are x[i] widened
 * exactly to binary32).  Each group of 256 consecutive elements is a
 * complete subtree.  The result is bit-identical for every block size,
 * chain length, grid and device, and n == 0 gives +0.0.  No MFMA is used.
 * Every node is one binary32 round-to-nearest-even addition: the first
 * level (two adjacent binary16 leaves) is computed by v_fma_mix_f32 as
 * lo * 1.0 + hi, whose product is exact and whose single rounding is that
 * of the binary32 sum, and every level above by v_add_f32.  This default
 * order is defined by IEEE arithmetic alone and is the one checked against
 * an emulation written from that definition.
 *
 * With ARMX_FLAG_MMA_LEAVES the prescribed order has tensor-core leaves (the
 * same Abstract reconstructs tensor-core arithmetic from outputs): x is cut
 * into chunks of 512 values (the last padded with -0.0), each chunk is one
 * v_mfma_f32_16x16x32_f16 against all-ones from a zero accumulator --
 * column j sums, in K order, values 8s .. 8s + 7 of the slots s = j, j + 16,
 * j + 32, j + 48 -- and the chunk's node is the balanced tree over its 16
 * column sums in column order; above the chunks the balanced tree as
 * before.  It is bit-identical for every block size, chain length and grid
 * on MI355X (gfx950).  What an MFMA leaf evaluates to is not specified by
 * any public document: this order's expected bits come from a model of the
 * gfx950 MFMA's accumulation that was fitted to, and checked against,
 * outputs of that hardware (oracle/mfma_model.py).  Agreement with it is
 * agreement with a model of one chip, not with IEEE arithmetic; the default
 * order above is the one pinned to arithmetic alone.
 *
 * x, n, out, ws, ws_bytes as for reduce_sum.  block_threads must be a power
 * of two.  ARMX_FLAG_PLAIN and ARMX_FLAG_ONE_CHAIN are not accepted.
 * Returns ARMX_OK or ARMX_ERR_{NULL,ALIGN,CONFIG,WORKSPACE,SHAPE,HIP}.
 */
int reduce_sum_fixed_order(const void* x, size_t n, float* out, void* ws,
                           size_t ws_bytes, const armx_config* cfg, void* stream);

/*
 * reduce_rows_fixed_order -- out[r] = the balanced-tree sum of row r.
 *
 *   "Taming Bitwise Behavior in GPU Kernels with Tensor Core", Abstract:
 *   tile shapes chosen for speed fix the arithmetic and can break batch
 *   invariance; a balanced-tree order makes a reduction reproducible.
 *
 * Row r's result is the root of the balanced binary tree over its cols
 * values x[r * ld + c] (padded with -0.0 to the next power of two, every
 * node one binary32 round-to-nearest-even addition) -- exactly
 * reduce_sum_fixed_order of that row alone.  It therefore depends on the
 * row's values only: not on rows, on the row's position, on the block size,
 * chain length or grid (batch invariance).  cols == 0 gives +0.0.
 *
 * With ARMX_FLAG_MMA_LEAVES every row is summed in the order with MFMA leaves
 * of reduce_sum_fixed_order instead: exactly reduce_sum_fixed_order of that
 * row alone with the flag, and batch invariant in the same way (its expected
 * bits rest on the same hardware-fitted model of the MFMA, see there).  Rows of at
 * most 512 values, several to a wavefront load, take one MFMA per lane block
 * with the other rows' lanes zeroed, so values never meet another row's.
 *
 * x, rows, cols, ld, out, ws as for reduce_rows (ld a multiple of 8 when
 * rows > 1).  With a workspace, few long rows are split into aligned
 * power-of-two chunk ranges (complete subtrees) over wavefronts of several
 * blocks, and the last block takes each row's tree over its ranges' roots;
 * and when a row stream's last round would be under three quarters full,
 * every row is split into two ranges in one launch (two rounds) or that
 * round's rows are split the same way in a second launch (more rounds).
 * All give the same bits as any other mapping.  block_threads must be a power of
 * two.  ARMX_FLAG_PLAIN, ARMX_FLAG_ONE_CHAIN and ARMX_FLAG_TWO_PASS are not
 * accepted.  Without a split (ws NULL, or enough rows), rows longer than the
 * LDS node logs allow (about 2^26 values at R = 8, 2^25 at the default
 * R = 4, 2^23 at R = 1) return ARMX_ERR_SHAPE.
 * Returns ARMX_OK or ARMX_ERR_{NULL,ALIGN,CONFIG,WORKSPACE,SHAPE,HIP}.
 */
int reduce_rows_fixed_order(const void* x, size_t rows, size_t cols, size_t ld, float* out,
                            void* ws, size_t ws_bytes, const armx_config* cfg, void* stream);

/*
 * reduce_sum_exact -- out[0] = the binary32 nearest (ties to even) to the
 * exact real sum of x[0..n); the same bits for every configuration.
 *
 *   The operation of "GPU Tensor Cores for fast Arithmetic Reductions",
 *   Abstract, without rounding error until the final 32-bit result: every
 *   binary16 value is an integer count of 2^-24, so the sum is kept as an
 *   integer split into two limbs with weights 1 and 2^32 -- components with
 *   fixed weights recombined exactly, as in "AWE: Adaptive Weight Encoding
 *   for Exact Integer Matrix Products with Fewer GEMMs on FP4 Tensor Cores"
 *   (arXiv 2609.24519), Abstract.  Integer addition is associative, so the
 *   result cannot depend on block size, chain length, grid or device, and it
 *   equals the correctly rounded sum.
 *
 * x, n, ws, ws_bytes, stream as for reduce_sum (the workspace holds 32 bytes
 * per block after its counter region).
 * out        device, 1 binary32.  n == 0, or an exact sum of zero, gives +0.0.
 * out_fixed  device, 2 int64 words, 8-byte aligned, or NULL: the exact sum
 *            as a 128-bit two's complement count of 2^-24 (out_fixed[0] the
 *            low 64 bits, out_fixed[1] the high 64 bits, signed); 0 when an
 *            input is an infinity or a NaN.
 * cfg        host, may be NULL.  Only ARMX_FLAG_CACHED_LOADS and
 *            ARMX_FLAG_INT_LIMBS are accepted.
 * By default each lane adds a chain's 8 R values in binary64 (exact: every
 * partial sum is a multiple of 2^-24 below 2^22), and the chain totals
 * accumulate as integers; no MFMA is used.  With ARMX_FLAG_INT_LIMBS every
 * value's count of 2^-24 is written as eight signed 8-bit digits (its limbs,
 * weights 2^(8m)), and v_mfma_i32_16x16x64_i8 against a digit-selector
 * operand sums each digit position exactly in 32-bit integers -- the integer
 * matrix cores do the additions -- before the positions are recombined with
 * their weights; same result bits, but about 14 vector instructions per
 * value to form the digits against 3 for the binary64 form, so it is bound
 * by the vector ALUs (measured on MI355X at 2^28 values: about 112 us
 * against 77 us); the binary64 form is the default for that reason.
 * Returns ARMX_OK or ARMX_ERR_{NULL,ALIGN,CONFIG,WORKSPACE,SHAPE,HIP}.
 */
int reduce_sum_exact(const void* x, size_t n, float* out, int64_t* out_fixed, void* ws,
                     size_t ws_bytes, const armx_config* cfg, void* stream);

/*
 * reduce_sum_noalloc -- reduce_sum without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 *
 * Same result, arguments and configuration as reduce_sum (the same bits as
 * reduce_sum with the same n, configuration and device), but the counter
 * region and block results live in a static device array of the library, 1
 * MiB per GPU, reserved when the library is loaded and held until the
 * process ends.  Each call first clears the counters its plan uses (a
 * 256-byte stretch per counter) with a small kernel on `stream`, then launches reduce_sum's kernels on it;
 * it calls no hipMalloc, hipFree or other allocating routine.  On its first
 * call on a device it looks up the array's device address
 * (hipGetSymbolAddress) with that device current.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one device (different streams, or graphs replayed concurrently) race and
 * must be serialised by the caller.
 * Returns ARMX_OK, ARMX_ERR_{NULL,ALIGN,CONFIG,SHAPE,HIP} as reduce_sum, or
 * ARMX_ERR_WORKSPACE when the configuration needs more than 1 MiB of
 * workspace (armx_workspace_bytes(ARMX_OP_SUM, ...) > 1048576: e.g. the
 * one-chain grid of ARMX_FLAG_ONE_CHAIN with small blocks and R on large
 * inputs, or ARMX_FLAG_MMA_LEVELS beyond about 2^30 values at R = 8).
 */
int reduce_sum_noalloc(const void* x, size_t n, float* out, const armx_config* cfg,
                       void* stream);

/* Operation codes for armx_workspace_bytes. */
#define ARMX_OP_SUM 0
#define ARMX_OP_ROWS 1
#define ARMX_OP_FIXED 2
#define ARMX_OP_ROWS_FIXED 3
#define ARMX_OP_EXACT 4

/*
 * armx_workspace_bytes -- bytes of workspace the matching call needs on the
 * current device with this configuration (0 if none).  `n_or_rows` is n for
 * ARMX_OP_SUM / ARMX_OP_FIXED / ARMX_OP_EXACT and rows for ARMX_OP_ROWS and
 * ARMX_OP_ROWS_FIXED; `cols` is used by those two only.  Returns (size_t)-1
 * for an invalid op or configuration.  Needs no GPU: without a device it
 * assumes 256 compute units.
 */
size_t armx_workspace_bytes(int op, size_t n_or_rows, size_t cols,
                            const armx_config* cfg);

/*
 * armx_launch_plan -- the launch shape the matching call would use on the
 * current device with this configuration (the same planning as the call
 * itself; nothing is enqueued, no device memory is touched).  Arguments as
 * for armx_workspace_bytes; `info` is a HOST pointer that receives:
 *   grid_blocks      blocks of the call's main (first) kernel launch
 *   block_threads    threads per block of that launch
 *   chain_r          16-byte loads per lane per loop step (R) of that launch
 *   waves_per_cu     resident wavefronts per compute unit that launch asks
 *                    for: grid_blocks * block_threads / 64 over the
 *                    compute-unit count (0 when nothing is launched)
 *   workspace_bytes  as armx_workspace_bytes
 *   lds_bytes        dynamic LDS per block of that launch
 *   launches         kernel launches the call enqueues
 * Without a device it assumes 256 compute units.  For the row operations
 * the plan is the one made with a workspace.  Returns ARMX_OK, or
 * ARMX_ERR_NULL (info NULL), ARMX_ERR_CONFIG or ARMX_ERR_SHAPE as the call
 * would.
 */
typedef struct armx_plan_info {
  int grid_blocks;
  int block_threads;
  int chain_r;
  double waves_per_cu;
  size_t workspace_bytes;
  size_t lds_bytes;
  int launches;
} armx_plan_info;

int armx_launch_plan(int op, size_t n_or_rows, size_t cols, const armx_config* cfg,
                     armx_plan_info* info);

/* armx_status_string -- a static, human-readable name for a status code. */
const char* armx_status_string(int status);

/* armx_version -- ABI version of this header: 8. */
int armx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ARMX_H */
