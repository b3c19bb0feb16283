// Producer step of a decode step: normalise, rotate, quantise and store the new tokens' K/V, fused.
//
// [P3] "Hy3 Preview AI Infra 推理优化精读笔记" §4.1: after the QKV projection, RoPE, RMSNorm,
// Hadamard, quantisation and the KV-cache write run as one kernel, keeping intermediates in
// registers and writing the cache directly in its low-bit format (§8: q and k are
// Hadamard-rotated before quantisation to spread outliers).  Per head vector x of 128 dims:
//   1. RMSNorm (optional): x / sqrt(mean(x^2) + eps) * w
//   2. RoPE (optional), rotate-half pairs (i, i + 64) turned by pos * theta^(-2i/128)
//   3. Hadamard (optional): Sylvester-ordered Walsh-Hadamard transform / sqrt(128)
// q takes 1-3 and is written back in bf16; k takes 1-3 and v none, and both go to the token's
// position in its request's paged cache (blocked layout of the attention kernels), as bf16 or as
// E4M3 codes of x / scale[head] (clamped to +-448, round to nearest even).
//
// gfx950 design: one wave per head vector (grid: B x 20 workgroups of 4 waves = the 64 q, 8 k and
// 8 v heads of a token), lane l holding dims l and l + 64 — exactly one RoPE pair — so RoPE is
// in-lane, the Hadamard's first stage (stride 64) is in-lane and its five other stages are lane
// exchanges, and the RMSNorm sum is one wave reduction.  The RoPE angle is formed in fp64 (a
// position of 2^17 times a frequency near 1 would lose ~0.01 rad in fp32) from frequencies the host
// computes once per call, and reduced mod 2 pi (one rint and one fma) before the fp32-accurate sine
// and cosine.  The work is a few hundred bytes per vector: the kernel is launch- and latency-bound.

#include <climits>
#include <cmath>

#include "common.h"
#include "lbsa.h"

namespace lbsa {

constexpr int kSD = 128;

struct StoreParams {
  const uint16_t* q_in;
  const uint16_t* k_in;
  const uint16_t* v_in;
  const float* q_norm_w;
  const float* k_norm_w;
  const int32_t* positions;
  uint16_t* q_out;
  uint8_t* k_cache;
  uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  int32_t bt_stride, num_pages, B, Hq, Hkv, page, fp8, hadamard;
  float eps, theta;
  double freq[kSD / 2];   // RoPE frequencies theta^(-2i/128), fp64, filled on the host
};

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  const __bf16 b = (__bf16)x;   // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += xor_lane(v, m);
  return v;
}

// E4M3 code of x (already clamped to +-448), round to nearest even (OCP E4M3 on gfx950)
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
  const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false);
  return (uint8_t)(packed & 0xff);
}

__global__ __launch_bounds__(256) void store_kv_kernel(StoreParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const int vec = blockIdx.y * 4 + wave;   // 0..Hq-1: q heads, then Hkv k heads, then Hkv v heads
  if (vec >= p.Hq + 2 * p.Hkv) return;
  const int kind = vec < p.Hq ? 0 : (vec < p.Hq + p.Hkv ? 1 : 2);
  const int head = kind == 0 ? vec : (kind == 1 ? vec - p.Hq : vec - p.Hq - p.Hkv);
  const int H = kind == 0 ? p.Hq : p.Hkv;
  const uint16_t* src = (kind == 0 ? p.q_in : (kind == 1 ? p.k_in : p.v_in)) + ((size_t)b * H + head) * kSD;
  float x0 = bf16_to_f32(src[lane]);
  float x1 = bf16_to_f32(src[lane + 64]);
  const int pos = p.positions[b];

  if (kind < 2) {
    const float* w = kind == 0 ? p.q_norm_w : p.k_norm_w;
    if (w) {
      const float ss = wave_sum_f32(x0 * x0 + x1 * x1);
      const float r = 1.0f / sqrtf(ss * (1.0f / kSD) + p.eps);
      x0 = x0 * r * w[lane];
      x1 = x1 * r * w[lane + 64];
    }
    if (p.theta > 0.f) {
      // angle = pos * theta^(-2 lane / 128) in fp64, reduced to [-pi, pi]
      constexpr double kTwoPi = 6.283185307179586476925286766559;
      double a = (double)pos * p.freq[lane];
      a = fma(-kTwoPi, rint(a * (1.0 / kTwoPi)), a);
      float s, c;
      sincosf((float)a, &s, &c);
      const float y0 = x0 * c - x1 * s;
      const float y1 = x1 * c + x0 * s;
      x0 = y0;
      x1 = y1;
    }
    if (p.hadamard) {
      // stride 64 in-lane, then strides 32 .. 1 across lanes: (u, v) -> (u + v, u - v)
      float y0 = x0 + x1, y1 = x0 - x1;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float o0 = xor_lane(y0, m), o1 = xor_lane(y1, m);
        const bool low = (lane & m) == 0;
        y0 = low ? y0 + o0 : o0 - y0;
        y1 = low ? y1 + o1 : o1 - y1;
      }
      const float norm = 0.08838834764831845f;   // 1 / sqrt(128)
      x0 = y0 * norm;
      x1 = y1 * norm;
    }
  }

  if (kind == 0) {
    uint16_t* dst = p.q_out + ((size_t)b * p.Hq + head) * kSD;
    dst[lane] = f32_to_bf16(x0);
    dst[lane + 64] = f32_to_bf16(x1);
    return;
  }

  // the cache slot of this token: page block_table[b][pos / page], offset pos % page; a position
  // or page id outside the table / cache is not stored
  if (pos < 0 || pos >= p.bt_stride * p.page) return;
  const int pid = p.block_table[(size_t)b * p.bt_stride + pos / p.page];
  if (pid < 0 || pid >= p.num_pages) return;
  const int t = pos % p.page;
  const int e = p.fp8 ? 1 : 2;
  const int w = 64 / e;   // elements per 64-byte row
  const size_t blk = ((size_t)pid * p.Hkv + head) * (size_t)p.page * kSD * e;
  const int d0 = lane, d1 = lane + 64;
  // K: [128 / w dim tiles][page][w]; V: [page / w token tiles][128][w]
  const size_t o0 = kind == 1 ? (size_t)((d0 / w) * p.page + t) * w + d0 % w : (size_t)((t / w) * kSD + d0) * w + t % w;
  const size_t o1 = kind == 1 ? (size_t)((d1 / w) * p.page + t) * w + d1 % w : (size_t)((t / w) * kSD + d1) * w + t % w;
  uint8_t* base = (kind == 1 ? p.k_cache : p.v_cache) + blk;
  if (p.fp8) {
    const float inv = 1.0f / (kind == 1 ? p.k_scale[head] : p.v_scale[head]);
    base[o0] = f32_to_e4m3(fminf(fmaxf(x0 * inv, -448.f), 448.f));
    base[o1] = f32_to_e4m3(fminf(fmaxf(x1 * inv, -448.f), 448.f));
  } else {
    reinterpret_cast<uint16_t*>(base)[o0] = f32_to_bf16(x0);
    reinterpret_cast<uint16_t*>(base)[o1] = f32_to_bf16(x1);
  }
}

}  // namespace lbsa

extern "C" int attn_store_kv(const void* q_in, const void* k_in, const void* v_in, const float* q_norm_w,
                             const float* k_norm_w, float norm_eps, const int32_t* positions, float rope_theta,
                             int32_t hadamard, void* q_out, void* k_cache, void* v_cache, int32_t kv_dtype,
                             const float* k_scale, const float* v_scale, const int32_t* block_table,
                             int32_t block_table_stride, int32_t num_pages, int32_t B, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t page_size, void* stream) {
  if (B < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_pages < 1 || block_table_stride < 0 || page_size < 1)
    return LBSA_ERR_INVALID;
  if (B == 0) return LBSA_OK;
  if (!q_in || !k_in || !v_in || !positions || !q_out || !k_cache || !v_cache || !block_table)
    return LBSA_ERR_INVALID;
  if (!(norm_eps >= 0.f) || !(rope_theta >= 0.f) || (hadamard != 0 && hadamard != 1)) return LBSA_ERR_INVALID;
  if (kv_dtype != LBSA_KV_BF16 && kv_dtype != LBSA_KV_FP8_E4M3) return LBSA_ERR_INVALID;
  if (kv_dtype == LBSA_KV_FP8_E4M3 && (!k_scale || !v_scale)) return LBSA_ERR_INVALID;
  if (head_dim != lbsa::kSD || page_size % 64 != 0) return LBSA_ERR_UNSUPPORTED;
  if ((int64_t)page_size * block_table_stride > INT32_MAX) return LBSA_ERR_INVALID;
  lbsa::StoreParams p{static_cast<const uint16_t*>(q_in), static_cast<const uint16_t*>(k_in),
                      static_cast<const uint16_t*>(v_in), q_norm_w, k_norm_w, positions,
                      static_cast<uint16_t*>(q_out), static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                      k_scale, v_scale, block_table, block_table_stride, num_pages, B, num_q_heads, num_kv_heads,
                      page_size, kv_dtype == LBSA_KV_FP8_E4M3 ? 1 : 0, hadamard, norm_eps, rope_theta, {}};
  for (int i = 0; i < lbsa::kSD / 2; ++i)
    p.freq[i] = rope_theta > 0.f ? std::pow((double)rope_theta, -2.0 * i / lbsa::kSD) : 0.0;
  const int vecs = num_q_heads + 2 * num_kv_heads;
  hipLaunchKernelGGL(lbsa::store_kv_kernel, dim3(B, (vecs + 3) / 4), dim3(256), 0, static_cast<hipStream_t>(stream),
                     p);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
