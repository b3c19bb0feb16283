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
// gfx950 design: a head vector is held by one row of 16 lanes, lane r keeping dims 4r..4r+3 and
// 64+4r..64+4r+3 — its four RoPE pairs — so RoPE is in-lane, loads and stores are 8-byte pieces
// (4-byte for E4M3 K), and of the Hadamard's seven stages three (strides 1, 2, 64) are in-lane and
// four (strides 4..32, lane bits 0..3) are DPP exchanges inside the 16-lane row; the RMSNorm sum is
// four more.  No LDS.  A wave holds four head vectors of one kind of one token (grid: B x ceil(20/4)
// workgroups of 4 waves for 64 q, 8 k and 8 v heads), which share the token's RoPE angles: lane l
// forms angle l in fp64 (a position of 2^17 times a frequency near 1 would lose ~0.01 rad in fp32)
// from frequencies the host computes once per call, reduces it mod 2 pi (one rint and one fma),
// takes the fp32-accurate sine and cosine, and the rows fetch theirs with lane permutes.  Every
// load of a wave is issued before the first wait.

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

__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const __bf16 b = (__bf16)x;   // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

// DPP moves inside a row of 16 lanes (all source lanes valid)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// value of lane (lane ^ M) of the same 16-lane row
template <int M>
__device__ __forceinline__ float row_xor(float x) {
  if constexpr (M == 1) return dpp<0xB1>(x);                 // quad_perm [1, 0, 3, 2]
  else if constexpr (M == 2) return dpp<0x4E>(x);            // quad_perm [2, 3, 0, 1]
  else if constexpr (M == 4) return dpp<0x141>(dpp<0x1B>(x));   // quad_perm [3, 2, 1, 0] then half-row mirror (^7)
  else return dpp<0x128>(x);                                 // row rotate by 8
}

// one Hadamard stage across lanes: (u, v) -> (u + v, u - v), u on the lane whose bit M is clear
template <int M>
__device__ __forceinline__ void lane_stage(float (&x)[8], int r) {
  const float sgn = (r & M) ? -1.f : 1.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = fmaf(sgn, x[j], row_xor<M>(x[j]));
}

// E4M3 code of x (already clamped to +-448), round to nearest even (OCP E4M3 on gfx950)
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
__device__ __forceinline__ uint8_t e4m3_one(float x) {
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xff);
}

__global__ __launch_bounds__(256) void store_kv_kernel(StoreParams p) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;   // lane within the vector's row: dims 4r..4r+3 and 64+4r..64+4r+3
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const int nq = (p.Hq + 3) >> 2, nk = (p.Hkv + 3) >> 2;
  const int task = blockIdx.y * 4 + wave;   // 4 heads of one kind: q blocks, then k blocks, then v blocks
  if (task >= nq + 2 * nk) return;
  const int kind = task < nq ? 0 : (task < nq + nk ? 1 : 2);
  const int hb = kind == 0 ? task : (kind == 1 ? task - nq : task - nq - nk);
  const int H = kind == 0 ? p.Hq : p.Hkv;
  const int head_raw = hb * 4 + (lane >> 4);
  const bool live = head_raw < H;
  const int head = live ? head_raw : H - 1;   // rows past the last head load a valid vector, store nothing

  // every load first
  const int pos = p.positions[b];
  const uint16_t* src = (kind == 0 ? p.q_in : (kind == 1 ? p.k_in : p.v_in)) + ((size_t)b * H + head) * kSD;
  const uint2 raw_lo = *reinterpret_cast<const uint2*>(src + 4 * r);
  const uint2 raw_hi = *reinterpret_cast<const uint2*>(src + 64 + 4 * r);
  const float* w = kind == 0 ? p.q_norm_w : (kind == 1 ? p.k_norm_w : nullptr);
  float4 w_lo = {}, w_hi = {};
  if (w) {
    w_lo = *reinterpret_cast<const float4*>(w + 4 * r);
    w_hi = *reinterpret_cast<const float4*>(w + 64 + 4 * r);
  }
  const bool rope = kind < 2 && p.theta > 0.f;
  const double freq = rope ? p.freq[lane] : 0.0;
  int pid = -1, t = 0;
  if (kind > 0 && pos >= 0 && pos < p.bt_stride * p.page) {
    pid = p.block_table[(size_t)b * p.bt_stride + pos / p.page];
    t = pos % p.page;
  }
  const float scale = kind > 0 && p.fp8 ? (kind == 1 ? p.k_scale : p.v_scale)[head] : 1.f;

  float x[8] = {bf16_lo(raw_lo.x), bf16_hi(raw_lo.x), bf16_lo(raw_lo.y), bf16_hi(raw_lo.y),
                bf16_lo(raw_hi.x), bf16_hi(raw_hi.x), bf16_lo(raw_hi.y), bf16_hi(raw_hi.y)};

  if (kind < 2) {
    if (w) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(x[j], x[j], ss);
      ss += row_xor<1>(ss);
      ss += row_xor<2>(ss);
      ss += row_xor<4>(ss);
      ss += row_xor<8>(ss);
      const float rn = 1.0f / sqrtf(ss * (1.0f / kSD) + p.eps);
      const float wv[8] = {w_lo.x, w_lo.y, w_lo.z, w_lo.w, w_hi.x, w_hi.y, w_hi.z, w_hi.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = x[j] * rn * wv[j];
    }
    if (rope) {
      // angle of pair `lane` = pos * theta^(-2 lane / 128) in fp64, reduced to [-pi, pi]
      constexpr double kTwoPi = 6.283185307179586476925286766559;
      double a = (double)pos * freq;
      a = fma(-kTwoPi, rint(a * (1.0 / kTwoPi)), a);
      float sn, cs;
      sincosf((float)a, &sn, &cs);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int from = (4 * r + j) << 2;   // pair 4r + j: dims (4r + j, 64 + 4r + j) = (x[j], x[4 + j])
        const float c = __int_as_float(__builtin_amdgcn_ds_bpermute(from, __float_as_int(cs)));
        const float s = __int_as_float(__builtin_amdgcn_ds_bpermute(from, __float_as_int(sn)));
        const float y0 = x[j] * c - x[4 + j] * s;
        const float y1 = x[4 + j] * c + x[j] * s;
        x[j] = y0;
        x[4 + j] = y1;
      }
    }
    if (p.hadamard) {
      // in-lane strides 1, 2 (dim bits 0, 1) and 64 (bit 6), then strides 4..32 over the row's lanes
#pragma unroll
      for (int h = 0; h < 8; h += 4) {
        float a0 = x[h] + x[h + 1], a1 = x[h] - x[h + 1], a2 = x[h + 2] + x[h + 3], a3 = x[h + 2] - x[h + 3];
        x[h] = a0 + a2;
        x[h + 1] = a1 + a3;
        x[h + 2] = a0 - a2;
        x[h + 3] = a1 - a3;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float u = x[j], v = x[4 + j];
        x[j] = u + v;
        x[4 + j] = u - v;
      }
      lane_stage<1>(x, r);
      lane_stage<2>(x, r);
      lane_stage<4>(x, r);
      lane_stage<8>(x, r);
      const float norm = 0.08838834764831845f;   // 1 / sqrt(128)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] *= norm;
    }
  }

  if (!live) return;
  if (kind == 0) {
    uint16_t* dst = p.q_out + ((size_t)b * p.Hq + head) * kSD;
    *reinterpret_cast<uint2*>(dst + 4 * r) = make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]));
    *reinterpret_cast<uint2*>(dst + 64 + 4 * r) = make_uint2(pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7]));
    return;
  }

  // the cache slot of this token: page block_table[b][pos / page], offset pos % page; a position
  // or page id outside the table / cache is not stored
  if (pid < 0 || pid >= p.num_pages) return;
  const size_t blk = ((size_t)pid * p.Hkv + head) * (size_t)p.page * kSD;   // elements of one (page, head) block
  if (p.fp8) {
    const float inv = 1.0f / scale;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = fminf(fmaxf(x[j] * inv, -448.f), 448.f);
    constexpr int wr = 64;   // codes per 64-byte row
    if (kind == 1) {
      // K: [2 dim tiles][page][64]; dims 4r..4r+3 in tile 0, 64+4r.. in tile 1
      uint8_t* k = p.k_cache + blk + (size_t)t * wr + 4 * r;
      *reinterpret_cast<uint32_t*>(k) = e4m3_pack4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<uint32_t*>(k + (size_t)p.page * wr) = e4m3_pack4(x[4], x[5], x[6], x[7]);
    } else {
      // V: [page / 64 token tiles][128][64]; each dim is its own 64-byte row
      uint8_t* v = p.v_cache + blk + (size_t)(t / wr) * kSD * wr + t % wr;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[(size_t)((j < 4 ? 4 * r : 60 + 4 * r) + j) * wr] = e4m3_one(x[j]);
    }
  } else {
    constexpr int wr = 32;   // bf16 elements per 64-byte row
    if (kind == 1) {
      // K: [4 dim tiles][page][32]; dims 4r..4r+3 in tile r / 8, 64+4r.. in tile 2 + r / 8
      uint16_t* k = reinterpret_cast<uint16_t*>(p.k_cache) + blk + (size_t)((r >> 3) * p.page + t) * wr + (4 * r) % wr;
      *reinterpret_cast<uint2*>(k) = make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]));
      *reinterpret_cast<uint2*>(k + (size_t)2 * p.page * wr) = make_uint2(pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7]));
    } else {
      // V: [page / 32 token tiles][128][32]
      uint16_t* v = reinterpret_cast<uint16_t*>(p.v_cache) + blk + (size_t)(t / wr) * kSD * wr + t % wr;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[(size_t)((j < 4 ? 4 * r : 60 + 4 * r) + j) * wr] = (uint16_t)f32_to_bf16(x[j]);
    }
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
  // 8-byte pieces of the vectors and caches, 16-byte pieces of the gains
  auto aligned = [](const void* ptr, uintptr_t a) { return ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % a == 0; };
  if (!aligned(q_in, 8) || !aligned(k_in, 8) || !aligned(v_in, 8) || !aligned(q_out, 8) || !aligned(k_cache, 8) ||
      !aligned(v_cache, 8) || !aligned(q_norm_w, 16) || !aligned(k_norm_w, 16))
    return LBSA_ERR_INVALID;
  if ((int64_t)page_size * block_table_stride > INT32_MAX) return LBSA_ERR_INVALID;
  lbsa::StoreParams p{static_cast<const uint16_t*>(q_in), static_cast<const uint16_t*>(k_in),
                      static_cast<const uint16_t*>(v_in), q_norm_w, k_norm_w, positions,
                      static_cast<uint16_t*>(q_out), static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                      k_scale, v_scale, block_table, block_table_stride, num_pages, B, num_q_heads, num_kv_heads,
                      page_size, kv_dtype == LBSA_KV_FP8_E4M3 ? 1 : 0, hadamard, norm_eps, rope_theta, {}};
  for (int i = 0; i < lbsa::kSD / 2; ++i)
    p.freq[i] = rope_theta > 0.f ? std::pow((double)rope_theta, -2.0 * i / lbsa::kSD) : 0.0;
  const int tasks = (num_q_heads + 3) / 4 + 2 * ((num_kv_heads + 3) / 4);   // 4 heads of one kind per wave
  hipLaunchKernelGGL(lbsa::store_kv_kernel, dim3(B, (tasks + 3) / 4), dim3(256), 0, static_cast<hipStream_t>(stream),
                     p);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
