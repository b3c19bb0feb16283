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

// WPI waves per (unit, row, query head) item.  Each lane owns two output dims and a wave walks the
// slots s = wave, wave + WPI, ... once, reading m, l and o together and keeping a running maximum
// (the online form of the definition above: the same sums, rescaled as the maximum grows), with
// four slots' loads in flight; with WPI > 1 the waves' states meet in LDS.  WPI = 1 serves units
// with a few slots (4 items per workgroup), WPI = 4 units split over many workers (one item per
// workgroup).
template <int WPI>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  __shared__ float2 red[WPI > 1 ? WPI * 64 : 1];
  __shared__ float2 red_ml[WPI > 1 ? WPI : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * (4 / WPI) + (WPI == 1 ? wave : 0);
  const int sub = WPI == 1 ? 0 : wave;
  const int64_t total = (int64_t)p.U * p.R * p.Hq;
  if (item >= total) return;
  // a device-built map that reported an error, or an unknown layout
  if (p.map[0] != LBSA_MAP_VERSION && p.map[0] != LBSA_MAP_VERSION_ORDERED && p.map[0] != LBSA_MAP_VERSION_PLACED)
    return;
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

  // one pass over the wave's slots s = sub, sub + WPI, ... with a running maximum M: the slot's
  // (m, l) are the same for every lane (each lane owns two output dims), so M, the rescaling and L
  // stay wave-uniform and need no lane reduction; four slots' loads are in flight at a time
  float M = -INFINITY, L = 0.f, a0 = 0.f, a1 = 0.f;
  // branch-free, so the loads of the next slots stay in flight: a slot with no visible key
  // (m = -inf) gets weight 0, and the running sums are rescaled by 0 when the first finite maximum
  // replaces -inf (they are still 0 then) and by 1 while the maximum is unchanged
  auto absorb = [&](float m, float l, float2 o) {
    const float Mn = fmaxf(M, m);
    const float sc = Mn == -INFINITY ? 1.f : fast_exp2((M - Mn) * kLog2e);
    const float w = m == -INFINITY ? 0.f : fast_exp2((m - Mn) * kLog2e);
    a0 = fmaf(w, o.x, a0 * sc);
    a1 = fmaf(w, o.y, a1 * sc);
    L = fmaf(w, l, L * sc);
    M = Mn;
  };
  int i = sub;
  for (; i + 3 * WPI < n; i += 4 * WPI) {
    float m[4], l[4];
    float2 o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[j] = p.part_m[slot(i + j * WPI)];
      l[j] = p.part_l[slot(i + j * WPI)];
      o[j] = *reinterpret_cast<const float2*>(p.part_o + slot(i + j * WPI) * 128 + 2 * lane);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) absorb(m[j], l[j], o[j]);
  }
  for (; i < n; i += WPI)
    absorb(p.part_m[slot(i)], p.part_l[slot(i)],
           *reinterpret_cast<const float2*>(p.part_o + slot(i) * 128 + 2 * lane));

  if constexpr (WPI > 1) {
    // merge the waves' running states: rescale each to the largest maximum
    red[wave * 64 + lane] = make_float2(a0, a1);
    if (lane == 0) red_ml[wave] = make_float2(M, L);
    __syncthreads();
    if (wave != 0) return;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPI; ++w) Mx = fmaxf(Mx, red_ml[w].x);
    a0 = 0.f;
    a1 = 0.f;
    L = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WPI; ++w) {
        const float2 ml = red_ml[w];
        if (ml.x == -INFINITY) continue;
        const float sc = fast_exp2((ml.x - Mx) * kLog2e);
        a0 += sc * red[w * 64 + lane].x;
        a1 += sc * red[w * 64 + lane].y;
        L += sc * ml.y;
      }
    }
  }
  if (L > 0.f) {
    const float inv = 1.f / L;
    a0 *= inv;
    a1 *= inv;
  } else {
    a0 = 0.f;   // a unit with no visible key
    a1 = 0.f;
  }
  const int64_t obase = (orow * p.Hq + h) * 128 + 2 * lane;
  if (p.out_bf16) {
    reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) + obase)[0] = pack_bf16(a0, a1);
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(p.out) + obase) = make_float2(a0, a1);
  }
}

// Row-wide form for units of many rows with 64 query heads (prefill): one workgroup per
// (unit, row), the four waves taking heads 16w .. 16w + 15 of the row.  A slot's partial row (64
// heads x 128 dims, 32 KiB) is read, and the output row written, with every load and store of a
// wave covering 1 KiB of contiguous bytes: lane l's k-th float4 is dims 4 (l % 32) .. +3 of head
// 16w + 2k + l / 32, so a lane keeps eight heads' running maxima and sums.  Two slots' loads are
// in flight at a time.
__global__ __launch_bounds__(256) void combine_rows_kernel(CombineParams p) {
  const int64_t ur = blockIdx.x;   // u * R + r
  const int t = threadIdx.x;
  const int wv = t >> 6;
  const int lane = t & 63;
  if (ur >= (int64_t)p.U * p.R) return;
  if (p.map[0] != LBSA_MAP_VERSION && p.map[0] != LBSA_MAP_VERSION_ORDERED && p.map[0] != LBSA_MAP_VERSION_PLACED)
    return;
  const int W = p.map[2];
  const int32_t* unit_ptr = p.map + 8 + (W + 1);
  const int32_t* units = unit_ptr + (p.U + 1);
  const int r = (int)(ur % p.R);
  const int u = (int)(ur / p.R);
  const int b = units[2 * u];
  const int qt = units[2 * u + 1];
  if (b < 0 || b >= p.map[1]) return;
  const int row_in_req = qt * p.R + r;
  if (row_in_req >= p.q_lens[b]) return;
  const int64_t orow = (int64_t)p.q_start[b] + row_in_req;
  const int s0 = unit_ptr[u];
  const int n = unit_ptr[u + 1] - s0;
  if (s0 < 0 || n < 0 || s0 + n > p.map[4]) return;
  const int h0 = 16 * wv + (lane >> 5);      // head of the lane's first float4; +2 per k
  const int q0 = 512 * wv + lane;            // float4 index of that float4 inside the row

  float M[8], L[8];
  f32x4 a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    M[k] = -INFINITY;
    L[k] = 0.f;
    a[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // the same branch-free online update as the per-head form, per head of the lane
  auto absorb = [&](const float (&m)[8], const float (&l)[8], const f32x4 (&o)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float Mn = fmaxf(M[k], m[k]);
      const float sc = Mn == -INFINITY ? 1.f : fast_exp2((M[k] - Mn) * kLog2e);
      const float w = m[k] == -INFINITY ? 0.f : fast_exp2((m[k] - Mn) * kLog2e);
      a[k] = w * o[k] + a[k] * sc;
      L[k] = fmaf(w, l[k], L[k] * sc);
      M[k] = Mn;
    }
  };
  auto load = [&](int i, float (&m)[8], float (&l)[8], f32x4 (&o)[8]) {
    const int64_t row = (int64_t)(s0 + i) * p.R + r;   // (slot, row) of the partials
    const f32x4* src = reinterpret_cast<const f32x4*>(p.part_o) + row * 2048 + q0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o[k] = src[64 * k];
      m[k] = p.part_m[row * 64 + h0 + 2 * k];
      l[k] = p.part_l[row * 64 + h0 + 2 * k];
    }
  };
  int i = 0;
  for (; i + 1 < n; i += 2) {
    float m0[8], l0[8], m1[8], l1[8];
    f32x4 o0[8], o1[8];
    load(i, m0, l0, o0);
    load(i + 1, m1, l1, o1);
    absorb(m0, l0, o0);
    absorb(m1, l1, o1);
  }
  if (i < n) {
    float m0[8], l0[8];
    f32x4 o0[8];
    load(i, m0, l0, o0);
    absorb(m0, l0, o0);
  }
  const int64_t obase = orow * 2048 + q0;   // float4 index
  if (p.out_bf16) {
    uint2* dst = reinterpret_cast<uint2*>(p.out) + obase;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float inv = L[k] > 0.f ? 1.f / L[k] : 0.f;   // a row with no visible key gets 0
      const f32x4 v = a[k] * inv;
      dst[64 * k] = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
  } else {
    f32x4* dst = reinterpret_cast<f32x4*>(p.out) + obase;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float inv = L[k] > 0.f ? 1.f / L[k] : 0.f;   // a row with no visible key gets 0
      dst[64 * k] = a[k] * inv;
    }
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
  if (q_lens && rows_per_unit >= 64 && num_q_heads == 64) {
    // units of many rows (prefill): one workgroup per (unit, row)
    const int64_t rows = (int64_t)num_units * rows_per_unit;
    if (rows > INT32_MAX) return LBSA_ERR_INVALID;
    if (reinterpret_cast<uintptr_t>(part_o) & 15 || reinterpret_cast<uintptr_t>(out) & (out_dtype ? 7 : 15))
      return LBSA_ERR_INVALID;
    hipLaunchKernelGGL(combine_rows_kernel, dim3((unsigned)rows), dim3(256), 0, st, p);
  } else if (max_splits > 16) {
    if (items > INT32_MAX) return LBSA_ERR_INVALID;
    hipLaunchKernelGGL(combine_kernel<4>, dim3((unsigned)items), dim3(256), 0, st, p);
  } else {
    const int64_t blocks = (items + 3) / 4;
    if (blocks > INT32_MAX) return LBSA_ERR_INVALID;
    hipLaunchKernelGGL(combine_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, p);
  }
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
