// Combine kernel: merges the split-KV partials of every query unit into the output
// ([P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案 step 5; [P4] §二.1: a combine kernel
// merges the split-KV results).
//
// Each thread owns four consecutive output dims of one (unit, row, query head); 32 threads
// cover the 128 dims.  The unit's slots are walked once with a running maximum:
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

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int W = p.map[2];
  const int32_t* unit_ptr = p.map + 8 + (W + 1);
  const int32_t* units = unit_ptr + (p.U + 1);
  const int64_t total = (int64_t)p.U * p.R * p.Hq * 32;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int d4 = (int)(idx & 31);
    int64_t rest = idx >> 5;
    const int h = (int)(rest % p.Hq);
    rest /= p.Hq;
    const int r = (int)(rest % p.R);
    const int u = (int)(rest / p.R);
    const int b = units[2 * u];
    const int qt = units[2 * u + 1];
    int64_t orow;
    if (p.q_lens) {
      const int row_in_req = qt * p.R + r;
      if (row_in_req >= p.q_lens[b]) continue;
      orow = (int64_t)p.q_start[b] + row_in_req;
    } else {
      orow = b;
    }
    float M = -INFINITY, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int s1 = unit_ptr[u + 1];
    for (int s = unit_ptr[u]; s < s1; ++s) {
      const int64_t slot = ((int64_t)s * p.R + r) * p.Hq + h;
      const float m = p.part_m[slot];
      if (m == -INFINITY) continue;
      if (m > M) {
        const float sc = fast_exp2((M - m) * kLog2e);   // M = -inf gives 0
        acc *= sc;
        L *= sc;
        M = m;
      }
      const float wgt = fast_exp2((m - M) * kLog2e);
      L += wgt * p.part_l[slot];
      const f32x4 o = *reinterpret_cast<const f32x4*>(p.part_o + slot * 128 + 4 * d4);
      acc += wgt * o;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    acc *= inv;
    const int64_t obase = (orow * p.Hq + h) * 128 + 4 * d4;
    if (p.out_bf16) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) + obase);
      dst[0] = pack_bf16(acc[0], acc[1]);
      dst[1] = pack_bf16(acc[2], acc[3]);
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase) = acc;
    }
  }
}

}  // namespace lbsa

using namespace lbsa;

extern "C" int attn_combine(const float* part_m, const float* part_l, const float* part_o,
                            const int32_t* map, int32_t num_units, int32_t rows_per_unit,
                            const int32_t* q_lens, const int32_t* q_start, int32_t num_q_heads,
                            int32_t head_dim, void* out, int32_t out_dtype, void* stream) {
  if (num_units < 0 || rows_per_unit < 1 || num_q_heads < 1 || !map || !out) return LBSA_ERR_INVALID;
  if ((q_lens == nullptr) != (q_start == nullptr)) return LBSA_ERR_INVALID;
  if (!q_lens && rows_per_unit != 1) return LBSA_ERR_INVALID;
  if (out_dtype != 0 && out_dtype != 1) return LBSA_ERR_INVALID;
  if (head_dim != 128) return LBSA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(part_o) | reinterpret_cast<uintptr_t>(out)) & (out_dtype ? 7 : 15))
    return LBSA_ERR_INVALID;
  if (num_units == 0) return LBSA_OK;
  CombineParams p{part_m, part_l, part_o, map, q_lens, q_start, out, num_units, rows_per_unit,
                  num_q_heads, out_dtype};
  const int64_t total = (int64_t)num_units * rows_per_unit * num_q_heads * 32;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
