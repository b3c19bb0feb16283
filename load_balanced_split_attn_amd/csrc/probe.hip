// Measurement probes, run beside the kernels: the device's practical HBM read ceiling and the rate
// its matrix cores sustain.
//
// Streaming read:
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

// Streaming read with per-XCD shares: workgroup b runs on XCD b mod 8 (the dispatcher's order).
// The buffer is cut into steps of UNROLL KiB, dealt to the XCDs in repeating cycles of
// L = q[0] + ... + q[7] steps, XCD x owning q[x] consecutive steps of each cycle; XCD x's waves take
// its steps in turn.  All XCDs move through the buffer together, as in stream_read_kernel, each at
// its own share; with q in proportion to the XCDs' streaming rates every XCD finishes at once, which
// equal shares do not give when the XCDs differ.  The sub-step tail is read by workgroup 0.
struct XcdShares {
  int32_t q[8];
};

template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_rated_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                                XcdShares sh, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int x = blockIdx.x & 7;
  const int64_t wx = (int64_t)(blockIdx.x >> 3) * 4 + (threadIdx.x >> 6);   // wave index inside XCD x
  const int64_t waves_x = (int64_t)(gridDim.x >> 3) * 4;
  int L = 0, pre = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pre += i < x ? sh.q[i] : 0;
    L += sh.q[i];
  }
  const int qx = sh.q[x];
  const int64_t step_elems = 64 * UNROLL;
  const int64_t n_steps = n16 / step_elems;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (qx > 0) {
    for (int64_t k = wx;; k += waves_x) {
      const int64_t c = k / qx;
      const int64_t step = c * L + pre + (k - c * qx);   // increases with k
      if (step >= n_steps) break;
      const u32x4* src = buf + step * step_elems + lane;
      u32x4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + 64 * u);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < 64)
    for (int64_t i = n_steps * step_elems + lane; i < n16; i += 64) acc ^= buf[i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Matrix-core rate: each wave issues `iters` rounds of eight independent v_mfma_f32_16x16x32_bf16
// products whose operands sit in registers (nothing is read from memory), so the launch measures the
// matrix pipes at the clock the chip holds while they run flat out.  The operands cycle over four
// register sets of random finite bf16 values (|x| in [0.5, 1)) so the multiplier inputs change on
// every product, as in a real contraction; eight accumulators put 128 cycles between dependent
// products, more than the instruction's latency.  The sum of a thread's accumulators goes to sink.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// The register budget is pinned (two waves per SIMD): left free, the compiler keeps the accumulators
// in AGPRs and copies them between register tuples on every round, which would time the copies.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_rate_kernel(
    int32_t iters, uint32_t* __restrict__ sink) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  u32x4 a[4], b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[k][e] = (probe_hash(t * 32u + 8u * k + e) & 0x807f807fu) | 0x3f003f00u;
      b[k][e] = (probe_hash(t * 32u + 8u * k + 4u + e) & 0x807f807fu) | 0x3f003f00u;
    }
  f32x4 c0{}, c1{}, c2{}, c3{}, c4{}, c5{}, c6{}, c7{};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma16x16x32(a[0], b[0], c0);
    c1 = mfma16x16x32(a[1], b[0], c1);
    c2 = mfma16x16x32(a[2], b[1], c2);
    c3 = mfma16x16x32(a[3], b[1], c3);
    c4 = mfma16x16x32(a[0], b[2], c4);
    c5 = mfma16x16x32(a[1], b[2], c5);
    c6 = mfma16x16x32(a[2], b[3], c6);
    c7 = mfma16x16x32(a[3], b[3], c7);
  }
  const f32x4 s4 = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  sink[t] = __float_as_uint((s4[0] + s4[1]) + (s4[2] + s4[3]));
}

}  // namespace lbsa

extern "C" int attn_probe_mfma_rate(int32_t iters, int32_t blocks, uint32_t* sink, void* stream) {
  if (!sink || iters < 1 || blocks < 1 || (reinterpret_cast<uintptr_t>(sink) & 3)) return LBSA_ERR_INVALID;
  hipLaunchKernelGGL(lbsa::mfma_rate_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}

extern "C" int attn_probe_stream_read_rated(const void* buf, int64_t bytes, int32_t blocks, const int32_t* xcd_rates,
                                            uint32_t* sink, void* stream) {
  if (!buf || !sink || !xcd_rates || bytes < 0 || (bytes & 15) || blocks < 8 || (blocks & 7) ||
      (reinterpret_cast<uintptr_t>(buf) & 15))
    return LBSA_ERR_INVALID;
  int32_t top = 0;
  for (int i = 0; i < 8; ++i) {
    if (xcd_rates[i] < 0 || xcd_rates[i] > LBSA_RATE_MAX) return LBSA_ERR_INVALID;
    top = xcd_rates[i] > top ? xcd_rates[i] : top;
  }
  if (top == 0) return LBSA_ERR_INVALID;
  // steps per cycle: the rates scaled so the fastest XCD owns 64 (a positive rate owns at least one)
  lbsa::XcdShares sh;
  for (int i = 0; i < 8; ++i) {
    const int64_t q = ((int64_t)xcd_rates[i] * 64 + top / 2) / top;
    sh.q[i] = xcd_rates[i] > 0 && q == 0 ? 1 : (int32_t)q;
  }
  hipLaunchKernelGGL(lbsa::stream_read_rated_kernel<LBSA_PROBE_UNROLL>, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const lbsa::u32x4*>(buf), bytes / 16, sh, sink);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}

extern "C" int attn_probe_stream_read(const void* buf, int64_t bytes, int32_t blocks, uint32_t* sink,
                                      void* stream) {
  if (!buf || !sink || bytes < 0 || (bytes & 15) || blocks < 1 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return LBSA_ERR_INVALID;
  hipLaunchKernelGGL(lbsa::stream_read_kernel<LBSA_PROBE_UNROLL>, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const lbsa::u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
