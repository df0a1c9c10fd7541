// Read-bandwidth probe (measurement only, libarmx_probe.so): the fastest a
// plain stream of 16-byte loads reads HBM on this device, with nothing but a
// XOR per loaded word (and, optionally, a pause of s_sleep `pause` after each
// step, the request pacing the reduction streams use).  The reductions are measured against its best launch
// shape as well as against the published peak.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "armx_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT, int PAUSE>
__global__ __launch_bounds__(1024) void read_probe_kernel(const u32x4* __restrict__ x,
                                                          uint64_t steps,
                                                          uint32_t* __restrict__ out) {
  const int lane = int(threadIdx.x) & 63;
  const uint64_t W = uint64_t(blockDim.x) >> 6;
  const uint64_t g = uint64_t(blockIdx.x) * W + (uint64_t(threadIdx.x) >> 6);
  const uint64_t T = uint64_t(gridDim.x) * W;
  uint32_t acc = 0;
  for (uint64_t s = g; s < steps; s += T) {
    const u32x4* p = x + s * (uint64_t(U) * 64) + lane;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (NT) {
        v[u] = __builtin_nontemporal_load(p + u * 64);
      } else {
        v[u] = p[u * 64];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    if constexpr (PAUSE > 0) __builtin_amdgcn_s_sleep(PAUSE);
  }
  out[g * 64 + uint64_t(lane)] = acc;
}

template <int U, int PAUSE>
const void* pick2(bool nt) {
  return nt ? reinterpret_cast<const void*>(&read_probe_kernel<U, true, PAUSE>)
            : reinterpret_cast<const void*>(&read_probe_kernel<U, false, PAUSE>);
}

template <int U>
const void* pick(bool nt, int pause) {
  switch (pause) {
    case 0: return pick2<U, 0>(nt);
    case 2: return pick2<U, 2>(nt);
    case 4: return pick2<U, 4>(nt);
    case 8: return pick2<U, 8>(nt);
    default: return nullptr;
  }
}

}  // namespace

extern "C" int armx_probe_read(const void* x, size_t n, uint32_t* out, size_t out_words,
                               int blocks, int block_threads, int loads, int nontemporal,
                               int pause, void* start_event, void* stop_event, void* stream) {
  if (!x || !out) return -1;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(out) % 4) return -2;
  if (blocks < 1 || block_threads < 64 || block_threads > 1024 || block_threads % 64) return -3;
  const void* fn = nullptr;
  const bool nt = nontemporal != 0;
  switch (loads) {
    case 1: fn = pick<1>(nt, pause); break;
    case 2: fn = pick<2>(nt, pause); break;
    case 4: fn = pick<4>(nt, pause); break;
    case 8: fn = pick<8>(nt, pause); break;
    case 16: fn = pick<16>(nt, pause); break;
    default: return -3;
  }
  if (!fn) return -3;
  const uint64_t per_step = uint64_t(loads) * 512;
  if (n == 0 || n % per_step) return -5;
  if (out_words < uint64_t(blocks) * uint64_t(block_threads)) return -5;
  const u32x4* xv = static_cast<const u32x4*>(x);
  uint64_t steps = n / per_step;
  void* args[] = {&xv, &steps, &out};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (start_event || stop_event) {
    e = hipExtLaunchKernel(fn, dim3(unsigned(blocks)), dim3(unsigned(block_threads)), args, 0, s,
                           static_cast<hipEvent_t>(start_event),
                           static_cast<hipEvent_t>(stop_event), 0);
  } else {
    e = hipLaunchKernel(fn, dim3(unsigned(blocks)), dim3(unsigned(block_threads)), args, 0, s);
  }
  return e == hipSuccess ? 0 : -6;
}
