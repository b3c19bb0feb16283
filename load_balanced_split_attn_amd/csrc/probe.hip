// Streaming-read probe: the device's practical HBM read ceiling, measured beside the kernels.
//
// Each wave reads UNROLL consecutive KiB (one 16-byte non-temporal load per lane per KiB) per step,
// steps spread over the grid; all loads of a step are issued before any is used.  Non-temporal
// loads of whole lines are the fastest plain read stream measured on gfx950 (~10% above default
// loads), so this is the ceiling a streaming kernel is compared with.
#include "common.h"
#include "lbsa.h"
#include "lbsa_probe.h"

#ifndef LBSA_PROBE_UNROLL
#define LBSA_PROBE_UNROLL 8
#endif

namespace lbsa {

template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int64_t step_elems = 64 * UNROLL;          // 16-byte elements per wave step
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t base = wave * step_elems;
  for (; base + step_elems <= n16; base += waves * step_elems) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(buf + base + 64 * u + lane);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (int64_t i = base + lane; i < n16 && i < base + step_elems; i += 64) acc ^= buf[i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace lbsa

extern "C" int attn_probe_stream_read(const void* buf, int64_t bytes, int32_t blocks, uint32_t* sink,
                                      void* stream) {
  if (!buf || !sink || bytes < 0 || (bytes & 15) || blocks < 1 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return LBSA_ERR_INVALID;
  hipLaunchKernelGGL(lbsa::stream_read_kernel<LBSA_PROBE_UNROLL>, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const lbsa::u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
