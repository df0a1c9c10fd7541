// Free-order sum: chained MFMAs against a ones operand (and the MFMA-free
// comparison design).
//
// "GPU Tensor Cores for fast Arithmetic Reductions" (arXiv 2001.05585),
// Abstract: the sum of n numbers is encoded as chains of m x m
// matrix-multiply-accumulates, each chain of R kept as a 32-bit float, and all
// chain results are reduced into one 32-bit float.  On gfx950 one chain step
// is v_mfma_f32_16x16x32_f16 with A = a 16 x 32 matrix of ones and B = the
// 32 x 16 tile a wavefront brings in with one 16-byte load per lane; R of
// them accumulate into the same fp32 registers.  By default A's lower 8 rows
// are -1 (the signed design, kSigned in device_common.hpp): half the
// accumulator elements carry the column sums and half their negations, and
// the total is half the difference, which cancels the downward lean of the
// MFMA's accumulation on wide-range data; ARMX_FLAG_ALL_ONES keeps A all
// ones.  The MFMA-free design ("conventional" reduction of the same Abstract)
// converts every value and adds it in fp32 per lane.
//
// Precision: every chain's R tile steps start from a zero fp32 accumulator,
// and the chain result is then added into a running fp32 sum, so the MFMA
// accumulates at most R x 32 values per column before its result is handed
// to a round-to-nearest-even add -- the chain sub-result of the Abstract.
//
// Work split: a "chain" is R consecutive chunks (R x 512 values).  Wavefront
// g of a grid of T wavefronts takes chains g, g + T, g + 2T, ...; the one
// partial chain at the end of the input (if any) is loaded with masking by
// the wavefront whose turn it is.  With a grid of ceil(chains / W) blocks
// every wavefront runs exactly one chain; smaller grids loop (persistent).
// Each block's wavefront totals are combined through LDS into one fp32 block
// result; a two-level completion ticket (groups of blocks, then the groups)
// lets the last block of each group and then the last group reduce the
// results in index order (or a second launch does, with ARMX_FLAG_TWO_PASS).
// No data atomics are used, so the result depends only on the configuration.
#include <atomic>
#include <mutex>

#include "device_common.hpp"
#include "launch.h"

namespace armx {
namespace {

using namespace dev;

static_assert(kTicketGroups == kMaxGroups && kTicketStride == kCounterStride &&
                  dev::kSplitCountRun == armx::kSplitCountRun,
              "the kernels' ticket layout is the plan's workspace layout");

// Reduces partials[0..count) in a fixed order with one block; valid in thread 0.
// A thread's values (i, i + B, ...) are added in that order, their loads
// issued four at a time so that they are in flight together (a loop of one
// load and one add waited a round trip per value: 2^24 values 10.09 -> 9.81
// us, 2^28 75.2 -> 75.0 us, the same bits).
__device__ float reduce_partials(const float* partials, unsigned count, float* red) {
  float s = 0.0f;
  const unsigned B = blockDim.x;
  unsigned i = threadIdx.x;
  for (; i + 3 * B < count; i += 4 * B) {
    const float a = load_published(partials + i), b = load_published(partials + i + B);
    const float c = load_published(partials + i + 2 * B), d = load_published(partials + i + 3 * B);
    s += a;
    s += b;
    s += c;
    s += d;
  }
  {
    const float a = i < count ? load_published(partials + i) : 0.0f;
    const float b = i + B < count ? load_published(partials + i + B) : 0.0f;
    const float c = i + 2 * B < count ? load_published(partials + i + 2 * B) : 0.0f;
    if (i < count) s += a;
    if (i + B < count) s += b;
    if (i + 2 * B < count) s += c;
  }
  s = wave_sum(s);
  return block_sum_lane0(s, red);
}

template <int R, bool NT, int D>
__global__ __launch_bounds__(1024) void sum_kernel(const u32x4* __restrict__ x, uint64_t n,
                                                   uint64_t chains_full,
                                                   unsigned* __restrict__ counters,
                                                   float* __restrict__ partials,
                                                   float* __restrict__ group_partials,
                                                   unsigned group, float* __restrict__ out,
                                                   int two_pass) {
  __shared__ float red[16];
  __shared__ int flag;
  const int lane = lane_id();
  const uint64_t W = uint64_t(num_waves());
  const uint64_t total_waves = uint64_t(gridDim.x) * W;
  uint64_t c = uint64_t(blockIdx.x) * W + uint64_t(wave_id());

  float run = 0.0f;
  const uint64_t iters = c < chains_full ? (chains_full - 1 - c) / total_waves + 1 : 0;
  // pacing (pace_pause), measured on MI355X: MFMA designs 8 from 64 chains
  // per wavefront, 2 from 8; MFMA-free design 4 from 64 chains
  constexpr bool PLAIN = D == kPlain;
  if (iters >= kPaceLongChains) {
    stream_chains<R, NT, D, PLAIN ? 4 : 8>(x, c, iters, total_waves, lane, run);
  } else if (!PLAIN && iters >= kPaceShortChains) {
    stream_chains<R, NT, D, 2>(x, c, iters, total_waves, lane, run);
  } else {
    stream_chains<R, NT, D>(x, c, iters, total_waves, lane, run);
  }
  c += iters * total_waves;
  if (c == chains_full && chains_full * R * 512 < n) {
    // the partial chain at the end: values past n read as +0.0
    tail_chain<R, D>(reinterpret_cast<const uint16_t*>(x), c, n, lane, run);
  }
  const float block_total = block_sum_lane0(wave_total<D>(run), red);

  if (gridDim.x == 1) {
    if (threadIdx.x == 0) out[0] = block_total;
    return;
  }
  if (two_pass) {
    if (threadIdx.x == 0) partials[blockIdx.x] = block_total;
    return;
  }
  finish_two_level(block_total, counters, partials, group_partials, group, out, red, &flag,
                   reduce_partials, chains_full < kSplitCountChains * total_waves);
}

__global__ __launch_bounds__(1024) void final_sum_kernel(const float* __restrict__ partials,
                                                         unsigned count,
                                                         float* __restrict__ out) {
  __shared__ float red[16];
  const float total = reduce_partials(partials, count, red);
  if (threadIdx.x == 0) out[0] = total;
}

__global__ void zero_kernel(float* out, uint64_t count) {
  const uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) out[i] = 0.0f;
}

template <int R, bool NT>
const void* pick_design(int d) {
  switch (d) {
    case kSigned: return reinterpret_cast<const void*>(&sum_kernel<R, NT, kSigned>);
    case kPlain: return reinterpret_cast<const void*>(&sum_kernel<R, NT, kPlain>);
    case kOnes: return reinterpret_cast<const void*>(&sum_kernel<R, NT, kOnes>);
    default: return nullptr;
  }
}

template <int R>
const void* pick_sum(bool nt, int d) {
  return nt ? pick_design<R, true>(d) : pick_design<R, false>(d);
}

const void* sum_kernel_for(int r, bool nt, int d) {
  switch (r) {
    case 1: return pick_sum<1>(nt, d);
    case 2: return pick_sum<2>(nt, d);
    case 3: return pick_sum<3>(nt, d);
    case 4: return pick_sum<4>(nt, d);
    case 5: return pick_sum<5>(nt, d);
    case 6: return pick_sum<6>(nt, d);
    case 7: return pick_sum<7>(nt, d);
    case 8: return pick_sum<8>(nt, d);
    default: return nullptr;
  }
}

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
std::mutex g_scratch_mutex;

}  // namespace

// Scratch memory of the allocation-free entry point (reduce_sum_noalloc): the
// counter region and block results that reduce_sum keeps in the caller's
// workspace, here in one static device array per GPU, held until the process
// ends.  Host code never passes `scratch` itself (in host code that name is a
// stand-in, not a device address): scratch_address() looks its device
// address up once per device with hipGetSymbolAddress and every use goes
// through that pointer.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_zero(float* out, uint64_t count, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  const unsigned blocks = unsigned((count + 255) / 256);
  void* args[] = {&out, &count};
  return hipLaunchKernel(reinterpret_cast<const void*>(&zero_kernel), dim3(blocks), dim3(256),
                         args, 0, stream);
}

hipError_t launch_sum(const Plan& plan, const void* x, float* out, void* ws, hipStream_t stream) {
  if (plan.n == 0) return launch_zero(out, 1, stream);
  const void* fn = sum_kernel_for(plan.r, (plan.flags & ARMX_FLAG_CACHED_LOADS) == 0,
                                  chain_design(plan.flags));
  if (!fn) return hipErrorInvalidValue;
  const u32x4* xv = static_cast<const u32x4*>(x);
  uint64_t n = plan.n;
  uint64_t chains_full = n / (uint64_t(plan.r) * kChunk);
  Workspace w = workspace_layout(plan, ws);
  unsigned group = plan.group;
  int two_pass = (plan.flags & ARMX_FLAG_TWO_PASS) ? 1 : 0;
  void* args[] = {&xv, &n, &chains_full, &w.counters, &w.partials, &w.group_partials, &group,
                  &out, &two_pass};
  hipError_t e = launch_main(plan, fn, args, stream);
  if (e != hipSuccess || !two_pass || plan.grid == 1) return e;
  unsigned count = unsigned(plan.grid);
  const float* cpart = w.partials;
  void* fargs[] = {&cpart, &count, &out};
  return hipLaunchKernel(reinterpret_cast<const void*>(&final_sum_kernel), dim3(1), dim3(1024),
                         fargs, 0, stream);
}

}  // namespace armx
