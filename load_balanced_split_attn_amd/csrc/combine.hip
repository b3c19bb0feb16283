// Combine kernel: merges the split-KV partials of every query unit into the output
// ([P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案 step 5; [P4] §二.1: a combine kernel
// merges the split-KV results).
//
// For every (unit, row, query head):
//   M = max_s m_s,  w_s = exp(m_s - M),  out = sum_s w_s o_s / sum_s w_s l_s,
// slots with m_s = -inf (no visible key) contribute nothing, and a unit with no visible key at
// all gets 0.  Slots of one unit are contiguous in the map, in ascending KV order.

#include "common.h"
#include "lbsa.h"

namespace lbsa {

struct CombineParams {
  const float* part_m;     // [S, R, Hq]
  const float* part_l;     // [S, R, Hq]
  const float* part_o;     // [S, R, Hq, 128]
  const int32_t* map;
  const int32_t* q_lens;   // prefill: rows of request b (null for decode)
  const int32_t* q_start;  // prefill: first output row of request b (null for decode)
  void* out;               // [rows, Hq, 128]
  int32_t U, R, Hq, out_bf16;
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, xor_lane(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += xor_lane(v, m);
  return v;
}

// WPI waves per (unit, row, query head) item.  Pass 1 spreads the unit's slots over the lanes for
// the maximum and the weighted sum of l (every wave of the item does it); pass 2 gives each lane two
// output dims and walks the slots s = wave, wave + WPI, ... with independent loads (unrolled), so
// the short, latency-bound loop keeps several in flight; with WPI > 1 the waves' sums meet in LDS.
// WPI = 1 serves units with a few slots (4 items per workgroup), WPI = 4 units split over many
// workers (one item per workgroup).
template <int WPI>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  __shared__ float2 red[WPI > 1 ? WPI * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * (4 / WPI) + (WPI == 1 ? wave : 0);
  const int sub = WPI == 1 ? 0 : wave;
  const int64_t total = (int64_t)p.U * p.R * p.Hq;
  if (item >= total) return;
  // a device-built map that reported an error, or an unknown layout
  if (p.map[0] != LBSA_MAP_VERSION && p.map[0] != LBSA_MAP_VERSION_ORDERED) return;
  const int W = p.map[2];
  const int32_t* unit_ptr = p.map + 8 + (W + 1);
  const int32_t* units = unit_ptr + (p.U + 1);
  const int h = (int)(item % p.Hq);
  const int64_t rest = item / p.Hq;
  const int r = (int)(rest % p.R);
  const int u = (int)(rest / p.R);
  const int b = units[2 * u];
  const int qt = units[2 * u + 1];
  // the map's own header bounds its requests and slots (the sizes the caller allocated from)
  if (b < 0 || b >= p.map[1]) return;
  int64_t orow;
  if (p.q_lens) {
    const int row_in_req = qt * p.R + r;
    if (row_in_req >= p.q_lens[b]) return;
    orow = (int64_t)p.q_start[b] + row_in_req;
  } else {
    orow = b;
  }
  const int s0 = unit_ptr[u];
  const int n = unit_ptr[u + 1] - s0;
  if (s0 < 0 || n < 0 || s0 + n > p.map[4]) return;
  auto slot = [&](int i) -> int64_t { return ((int64_t)(s0 + i) * p.R + r) * p.Hq + h; };

  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, p.part_m[slot(i)]);
  M = wave_max(M);
  float L = 0.f;
  if (M != -INFINITY) {
    for (int i = lane; i < n; i += 64) {
      const float m = p.part_m[slot(i)];
      if (m != -INFINITY) L += fast_exp2((m - M) * kLog2e) * p.part_l[slot(i)];
    }
  }
  L = wave_sum(L);

  float a0 = 0.f, a1 = 0.f;
  if (L > 0.f) {
    int i = sub;
    for (; i + 3 * WPI < n; i += 4 * WPI) {
      float m[4];
      float2 o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m[j] = p.part_m[slot(i + j * WPI)];
        o[j] = *reinterpret_cast<const float2*>(p.part_o + slot(i + j * WPI) * 128 + 2 * lane);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float w = (m[j] == -INFINITY) ? 0.f : fast_exp2((m[j] - M) * kLog2e);
        a0 += w * o[j].x;
        a1 += w * o[j].y;
      }
    }
    for (; i < n; i += WPI) {
      const float m = p.part_m[slot(i)];
      const float2 o = *reinterpret_cast<const float2*>(p.part_o + slot(i) * 128 + 2 * lane);
      const float w = (m == -INFINITY) ? 0.f : fast_exp2((m - M) * kLog2e);
      a0 += w * o.x;
      a1 += w * o.y;
    }
  }
  if constexpr (WPI > 1) {
    red[wave * 64 + lane] = make_float2(a0, a1);
    __syncthreads();
    if (wave != 0) return;
    a0 = 0.f;
    a1 = 0.f;
#pragma unroll
    for (int w = 0; w < WPI; ++w) {
      a0 += red[w * 64 + lane].x;
      a1 += red[w * 64 + lane].y;
    }
  }
  if (L > 0.f) {
    const float inv = 1.f / L;
    a0 *= inv;
    a1 *= inv;
  }
  const int64_t obase = (orow * p.Hq + h) * 128 + 2 * lane;
  if (p.out_bf16) {
    reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) + obase)[0] = pack_bf16(a0, a1);
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(p.out) + obase) = make_float2(a0, a1);
  }
}

}  // namespace lbsa

using namespace lbsa;

extern "C" int attn_combine(const float* part_m, const float* part_l, const float* part_o,
                            const int32_t* map, int32_t num_units, int32_t rows_per_unit,
                            const int32_t* q_lens, const int32_t* q_start, int32_t num_q_heads,
                            int32_t head_dim, void* out, int32_t out_dtype, int32_t max_splits,
                            void* stream) {
  if (num_units < 0 || rows_per_unit < 1 || num_q_heads < 1 || !map || !out || max_splits < 0)
    return LBSA_ERR_INVALID;
  if ((q_lens == nullptr) != (q_start == nullptr)) return LBSA_ERR_INVALID;
  if (!q_lens && rows_per_unit != 1) return LBSA_ERR_INVALID;
  if (out_dtype != 0 && out_dtype != 1) return LBSA_ERR_INVALID;
  if (head_dim != 128) return LBSA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(part_o) | reinterpret_cast<uintptr_t>(out)) & (out_dtype ? 3 : 7))
    return LBSA_ERR_INVALID;
  if (num_units == 0) return LBSA_OK;
  CombineParams p{part_m, part_l, part_o, map, q_lens, q_start, out, num_units, rows_per_unit,
                  num_q_heads, out_dtype};
  const int64_t items = (int64_t)num_units * rows_per_unit * num_q_heads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (max_splits > 16) {
    if (items > INT32_MAX) return LBSA_ERR_INVALID;
    hipLaunchKernelGGL(combine_kernel<4>, dim3((unsigned)items), dim3(256), 0, st, p);
  } else {
    const int64_t blocks = (items + 3) / 4;
    if (blocks > INT32_MAX) return LBSA_ERR_INVALID;
    hipLaunchKernelGGL(combine_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, p);
  }
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
