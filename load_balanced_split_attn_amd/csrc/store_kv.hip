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
// forms angle l in turns in fp64 (a position of 2^17 times a frequency near 1 would lose ~0.01 rad
// in fp32) from frequencies the host computes once per call, reduces it to [-1/2, 1/2] turn (one
// rint), takes the hardware sine and cosine of the reduced turn, and the rows fetch theirs with lane
// permutes.  Every load of a wave is issued before the first wait.  A prefill chunk
// (attn_store_kv_chunk) runs one workgroup per new row whose waves loop over the q and k head
// groups with the row's angles formed once, and writes V through a separate kernel in whole
// 64-byte cache rows.

#include <climits>
#include <cmath>

#include "common.h"
#include "lbsa.h"

namespace lbsa {

constexpr int kSD = 128;

struct StoreParams {
  // chunk append (attn_store_kv_chunk): request b's q_lens[b] new rows start at row q_start[b] and
  // take positions positions[b] + j; null for the one-token step, where row b is request b's token
  const int32_t* q_lens;
  const int32_t* q_start;
  int32_t max_rows;   // chunk append: rows per request the grid covers (>= every q_lens[b])
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
  double freq[kSD / 2];   // RoPE frequencies theta^(-2i/128) in turns (divided by 2 pi), fp64, filled on the host
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

// RoPE sine and cosine of pair `lane` (pairs 0..63) at position pos.  The angle pos * theta^(-2 lane
// / 128) is formed in turns and reduced to [-1/2, 1/2] in fp64 (a position of 2^17 times a frequency
// near 1 would lose ~0.01 rad in fp32); the hardware sine and cosine of the reduced turn follow.
__device__ __forceinline__ void rope_angle(const StoreParams& p, int lane, int pos, float& sn, float& cs) {
  double turns = (double)pos * p.freq[lane];
  turns -= rint(turns);
  const float f = (float)turns;
  sn = __builtin_amdgcn_sinf(f);   // sin(2 pi f)
  cs = __builtin_amdgcn_cosf(f);
}

// One task: four head vectors of one kind (task < nq: q heads 4 task ..; then k; then v) of one
// token, one per 16-lane row of the wave.  Rows past the last head take the last head's vector and
// store nothing.
struct TaskHead {
  int kind;   // 0 q, 1 k, 2 v
  int head;
  bool live;
};
__device__ __forceinline__ TaskHead task_head(const StoreParams& p, int task, int nq, int nk, int lane) {
  const int kind = task < nq ? 0 : (task < nq + nk ? 1 : 2);
  const int hb = kind == 0 ? task : (kind == 1 ? task - nq : task - nq - nk);
  const int H = kind == 0 ? p.Hq : p.Hkv;
  const int head_raw = hb * 4 + (lane >> 4);
  return TaskHead{kind, head_raw < H ? head_raw : H - 1, head_raw < H};
}

// The lane's pieces of its head vector in `row` (dims 4r..4r+3 and 64+4r..64+4r+3, bf16 pairs) and,
// for k and v over an 8-bit cache, the head's scale (1 otherwise).
struct TaskIn {
  uint2 lo, hi;
  float scale;
};
__device__ __forceinline__ TaskIn load_task(const StoreParams& p, const TaskHead& th, int row, int r) {
  const int H = th.kind == 0 ? p.Hq : p.Hkv;
  const uint16_t* src = (th.kind == 0 ? p.q_in : (th.kind == 1 ? p.k_in : p.v_in)) + ((size_t)row * H + th.head) * kSD;
  const float scale = th.kind > 0 && p.fp8 ? (th.kind == 1 ? p.k_scale : p.v_scale)[th.head] : 1.f;
  return TaskIn{*reinterpret_cast<const uint2*>(src + 4 * r), *reinterpret_cast<const uint2*>(src + 64 + 4 * r), scale};
}

// RMSNorm gains of the lane's dims (zeros when w is null: no norm)
struct Gains {
  float4 lo, hi;
};
__device__ __forceinline__ Gains load_gains(const float* w, int r) {
  if (!w) return Gains{};
  return Gains{*reinterpret_cast<const float4*>(w + 4 * r), *reinterpret_cast<const float4*>(w + 64 + 4 * r)};
}

// Cache slot of the token at pos in request b: page block_table[b][pos / page] and offset pos % page;
// pid = -1 for a position outside the table (not stored)
__device__ __forceinline__ void cache_slot(const StoreParams& p, int b, int pos, int& pid, int& t) {
  pid = -1;
  t = 0;
  if (pos >= 0 && pos < p.bt_stride * p.page) {
    pid = p.block_table[(size_t)b * p.bt_stride + pos / p.page];
    t = pos % p.page;
  }
}

// The arithmetic and the stores of one task whose loads (vector, gains, cache slot) are done; RoPE
// angles (sn, cs) of pair `lane` already formed.  norm: the task's kind has RMSNorm gains.
__device__ __forceinline__ void store_task(const StoreParams& p, const TaskHead& th, const TaskIn& in, bool norm,
                                           const Gains& gn, int row, int pid, int t, float sn, float cs) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;   // lane within the vector's row: dims 4r..4r+3 and 64+4r..64+4r+3
  const int kind = th.kind, head = th.head;
  const bool rope = kind < 2 && p.theta > 0.f;
  const uint2 raw_lo = in.lo, raw_hi = in.hi;
  const float4 w_lo = gn.lo, w_hi = gn.hi;
  const float scale = in.scale;

  float x[8] = {bf16_lo(raw_lo.x), bf16_hi(raw_lo.x), bf16_lo(raw_lo.y), bf16_hi(raw_lo.y),
                bf16_lo(raw_hi.x), bf16_hi(raw_hi.x), bf16_lo(raw_hi.y), bf16_hi(raw_hi.y)};

  if (kind < 2) {
    if (norm) {
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

  if (!th.live) return;
  if (kind == 0) {
    uint16_t* dst = p.q_out + ((size_t)row * p.Hq + head) * kSD;
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

// CHUNK = false: one new token per request, row b at positions[b]; one task (q, k or v heads) per
// wave, every load issued before the arithmetic.  CHUNK = true: request b's q_lens[b] rows from row
// q_start[b] at positions positions[b] + j; one workgroup per row, each wave looping over every
// fourth q/k task with the row's RoPE angles, gains and cache slot formed once, and the next task's
// loads in flight while the current task is computed (the chunk's V goes through
// store_v_chunk_kernel, which writes whole 64-byte rows).
template <bool CHUNK>
__global__ __launch_bounds__(256) void store_kv_kernel(StoreParams p) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nq = (p.Hq + 3) >> 2, nk = (p.Hkv + 3) >> 2;
  const bool rope = p.theta > 0.f;
  float sn = 0.f, cs = 1.f;
  if constexpr (CHUNK) {
    const int b = blockIdx.x / p.max_rows;
    const int j = blockIdx.x - b * p.max_rows;
    if (j >= p.q_lens[b]) return;
    const int ntask = nq + nk;
    int task = wave;
    if (task >= ntask) return;
    const int row = p.q_start[b] + j;
    const int pos = p.positions[b] < 0 ? -1 : p.positions[b] + j;   // a chunk starting before 0 is not stored
    int pid, t;
    cache_slot(p, b, pos, pid, t);
    if (rope) rope_angle(p, lane, pos, sn, cs);
    for (; task < ntask; task += 4) {
      const TaskHead th = task_head(p, task, nq, nk, lane);
      const TaskIn in = load_task(p, th, row, r);
      const float* w = th.kind == 0 ? p.q_norm_w : p.k_norm_w;
      const Gains gn = load_gains(w, r);
      store_task(p, th, in, w != nullptr, gn, row, pid, t, sn, cs);
    }
  } else {
    const int b = blockIdx.x;
    const int pos = p.positions[b];
    const int task = blockIdx.y * 4 + wave;   // 4 heads of one kind: q blocks, then k blocks, then v blocks
    if (task >= nq + 2 * nk) return;
    const TaskHead th = task_head(p, task, nq, nk, lane);
    const TaskIn in = load_task(p, th, b, r);
    const float* w = th.kind == 0 ? p.q_norm_w : (th.kind == 1 ? p.k_norm_w : nullptr);
    const Gains gn = load_gains(w, r);
    int pid = -1, t = 0;
    if (th.kind > 0) cache_slot(p, b, pos, pid, t);
    if (rope && th.kind < 2) rope_angle(p, lane, pos, sn, cs);
    store_task(p, th, in, w != nullptr, gn, b, pid, t, sn, cs);
  }
}

// V of a chunk append: one workgroup per (request, 64-byte-row token tile, KV head) writes whole rows.
// The blocked cache keeps V dim-major inside tiles of TT tokens (TT = 32 bf16 or 64 E4M3 codes per
// 64-byte row), so appending one token touches 128 separate rows; a chunk of consecutive tokens
// fills them.  The tile's tokens are staged in LDS token-major, then each thread writes 32 bytes of
// one dim row.  Tokens of the tile outside the chunk (the cached prefix before it, free slots after
// it) keep the bytes the cache holds: the edge tiles read their rows first and merge.
template <bool FP8>
__global__ __launch_bounds__(256) void store_v_chunk_kernel(StoreParams p, int tiles_per_request) {
  constexpr int TT = FP8 ? 64 : 32;   // tokens per 64-byte V row
  constexpr int kPad = 8;             // bf16 elements of padding per staged token row
  __shared__ __attribute__((aligned(16))) uint16_t sv[TT][kSD + kPad];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / tiles_per_request;
  const int jt = blockIdx.x - b * tiles_per_request;
  const int g = blockIdx.y;
  const int n = p.q_lens[b];
  const int pos0 = p.positions[b];
  if (n <= 0 || pos0 < 0) return;
  const int T0 = (pos0 / TT + jt) * TT;           // first token of this workgroup's tile
  const int lo = max(T0, pos0), hi = min(T0 + TT, pos0 + n);
  if (lo >= hi || T0 >= p.bt_stride * p.page) return;
  const int pid = p.block_table[(size_t)b * p.bt_stride + T0 / p.page];
  if (pid < 0 || pid >= p.num_pages) return;
  const int row0 = p.q_start[b] - pos0;            // q/k/v row of token t is row0 + t

  // stage the tile's tokens (zeros outside [lo, hi)): TT tokens x 16 granules of 16 bytes
#pragma unroll
  for (int i = tid; i < TT * 16; i += 256) {
    const int tok = i >> 4, gr = i & 15, t = T0 + tok;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (t >= lo && t < hi) val = *reinterpret_cast<const uint4*>(p.v_in + ((size_t)(row0 + t) * p.Hkv + g) * kSD + 8 * gr);
    *reinterpret_cast<uint4*>(&sv[tok][8 * gr]) = val;
  }
  __syncthreads();

  // thread -> dim row d, half h of the row (TT / 2 tokens, 32 bytes)
  const int d = tid >> 1, h = tid & 1;
  const int tok_base = h * (TT / 2);
  const size_t blk = ((size_t)pid * p.Hkv + g) * (size_t)p.page * kSD;   // elements of one (page, head) block
  const int tile_in_page = (T0 % p.page) / TT;
  const size_t row_off = blk + ((size_t)tile_in_page * kSD + d) * TT + tok_base;   // elements
  const bool edge = lo > T0 || hi < T0 + TT;
  if constexpr (FP8) {
    uint8_t* dst = p.v_cache + row_off;
    const float inv = 1.0f / p.v_scale[g];
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t bits = sv[tok_base + 4 * k + e][d];
        x[e] = fminf(fmaxf(__uint_as_float((uint32_t)bits << 16) * inv, -448.f), 448.f);
      }
      w[k] = e4m3_pack4(x[0], x[1], x[2], x[3]);
    }
    if (edge) {
      const uint4 old0 = *reinterpret_cast<const uint4*>(dst), old1 = *reinterpret_cast<const uint4*>(dst + 16);
      const uint32_t o[8] = {old0.x, old0.y, old0.z, old0.w, old1.x, old1.y, old1.z, old1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint32_t keep = 0u;   // byte lanes of tokens outside the chunk keep the cache's bytes
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = T0 + tok_base + 4 * k + e;
          if (t < lo || t >= hi) keep |= 0xffu << (8 * e);
        }
        w[k] = (w[k] & ~keep) | (o[k] & keep);
      }
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(p.v_cache) + row_off;
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = (uint32_t)sv[tok_base + 2 * k][d] | ((uint32_t)sv[tok_base + 2 * k + 1][d] << 16);
    if (edge) {
      const uint4 old0 = *reinterpret_cast<const uint4*>(dst), old1 = *reinterpret_cast<const uint4*>(dst + 8);
      const uint32_t o[8] = {old0.x, old0.y, old0.z, old0.w, old1.x, old1.y, old1.z, old1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int t = T0 + tok_base + 2 * k;
        const uint32_t keep = ((t < lo || t >= hi) ? 0x0000ffffu : 0u) | ((t + 1 < lo || t + 1 >= hi) ? 0xffff0000u : 0u);
        w[k] = (w[k] & ~keep) | (o[k] & keep);
      }
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// Host-side checks shared by both entry points; fills p except the chunk fields.
static int store_setup(StoreParams& p, const void* q_in, const void* k_in, const void* v_in, const float* q_norm_w,
                       const float* k_norm_w, float norm_eps, const int32_t* positions, float rope_theta,
                       int32_t hadamard, void* q_out, void* k_cache, void* v_cache, int32_t kv_dtype,
                       const float* k_scale, const float* v_scale, const int32_t* block_table,
                       int32_t block_table_stride, int32_t num_pages, int32_t B, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size) {
  if (B < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_pages < 1 || block_table_stride < 0 || page_size < 1)
    return LBSA_ERR_INVALID;
  if (!q_in || !k_in || !v_in || !positions || !q_out || !k_cache || !v_cache || !block_table)
    return LBSA_ERR_INVALID;
  if (!(norm_eps >= 0.f) || !(rope_theta >= 0.f) || (hadamard != 0 && hadamard != 1)) return LBSA_ERR_INVALID;
  if (kv_dtype != LBSA_KV_BF16 && kv_dtype != LBSA_KV_FP8_E4M3) return LBSA_ERR_INVALID;
  if (kv_dtype == LBSA_KV_FP8_E4M3 && (!k_scale || !v_scale)) return LBSA_ERR_INVALID;
  if (head_dim != kSD || page_size % 64 != 0) return LBSA_ERR_UNSUPPORTED;
  // 8-byte pieces of the vectors and caches, 16-byte pieces of the gains
  auto aligned = [](const void* ptr, uintptr_t a) { return ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % a == 0; };
  if (!aligned(q_in, 8) || !aligned(k_in, 8) || !aligned(v_in, 8) || !aligned(q_out, 8) || !aligned(k_cache, 8) ||
      !aligned(v_cache, 8) || !aligned(q_norm_w, 16) || !aligned(k_norm_w, 16))
    return LBSA_ERR_INVALID;
  if ((int64_t)page_size * block_table_stride > INT32_MAX) return LBSA_ERR_INVALID;
  p = StoreParams{nullptr, nullptr, 0, static_cast<const uint16_t*>(q_in), static_cast<const uint16_t*>(k_in),
                  static_cast<const uint16_t*>(v_in), q_norm_w, k_norm_w, positions,
                  static_cast<uint16_t*>(q_out), static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                  k_scale, v_scale, block_table, block_table_stride, num_pages, B, num_q_heads, num_kv_heads,
                  page_size, kv_dtype == LBSA_KV_FP8_E4M3 ? 1 : 0, hadamard, norm_eps, rope_theta, {}};
  for (int i = 0; i < kSD / 2; ++i)
    p.freq[i] = rope_theta > 0.f ? std::pow((double)rope_theta, -2.0 * i / kSD) / (2.0 * M_PI) : 0.0;
  return LBSA_OK;
}

}  // namespace lbsa

extern "C" int attn_store_kv(const void* q_in, const void* k_in, const void* v_in, const float* q_norm_w,
                             const float* k_norm_w, float norm_eps, const int32_t* positions, float rope_theta,
                             int32_t hadamard, void* q_out, void* k_cache, void* v_cache, int32_t kv_dtype,
                             const float* k_scale, const float* v_scale, const int32_t* block_table,
                             int32_t block_table_stride, int32_t num_pages, int32_t B, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t page_size, void* stream) {
  if (B == 0 && num_q_heads >= 1 && num_kv_heads >= 1 && num_pages >= 1 && block_table_stride >= 0 && page_size >= 1)
    return LBSA_OK;
  lbsa::StoreParams p;
  const int rc = lbsa::store_setup(p, q_in, k_in, v_in, q_norm_w, k_norm_w, norm_eps, positions, rope_theta, hadamard,
                                   q_out, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table,
                                   block_table_stride, num_pages, B, num_q_heads, num_kv_heads, head_dim, page_size);
  if (rc != LBSA_OK) return rc;
  const int tasks = (num_q_heads + 3) / 4 + 2 * ((num_kv_heads + 3) / 4);   // 4 heads of one kind per wave
  hipLaunchKernelGGL(lbsa::store_kv_kernel<false>, dim3(B, (tasks + 3) / 4), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}

extern "C" int attn_store_kv_chunk(const void* q_in, const void* k_in, const void* v_in, const float* q_norm_w,
                                   const float* k_norm_w, float norm_eps, const int32_t* q_lens,
                                   const int32_t* q_start, const int32_t* positions, int32_t max_q_len,
                                   float rope_theta, int32_t hadamard, void* q_out, void* k_cache, void* v_cache,
                                   int32_t kv_dtype, const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                                   int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t page_size, void* stream) {
  if (max_q_len < 0 || !q_lens || !q_start) return LBSA_ERR_INVALID;
  lbsa::StoreParams p;
  const int rc = lbsa::store_setup(p, q_in, k_in, v_in, q_norm_w, k_norm_w, norm_eps, positions, rope_theta, hadamard,
                                   q_out, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table,
                                   block_table_stride, num_pages, B, num_q_heads, num_kv_heads, head_dim, page_size);
  if (rc != LBSA_OK) return rc;
  if (B == 0 || max_q_len == 0) return LBSA_OK;
  // V rows are 16-byte pieces of 128-dim vectors in the staging loads
  if ((reinterpret_cast<uintptr_t>(v_in) | reinterpret_cast<uintptr_t>(v_cache)) & 15) return LBSA_ERR_INVALID;
  p.q_lens = q_lens;
  p.q_start = q_start;
  p.max_rows = max_q_len;
  const int64_t qk_blocks = (int64_t)B * max_q_len;
  const int tt = p.fp8 ? 64 : 32;
  const int64_t tiles = (max_q_len + tt - 1) / tt + 1;   // a chunk starting inside a tile covers one more
  if (qk_blocks > INT32_MAX || (int64_t)B * tiles > INT32_MAX) return LBSA_ERR_INVALID;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(lbsa::store_kv_kernel<true>, dim3((unsigned)qk_blocks), dim3(256), 0, st, p);   // q and k; V below
  if (p.fp8)
    hipLaunchKernelGGL(lbsa::store_v_chunk_kernel<true>, dim3((unsigned)(B * tiles), num_kv_heads), dim3(256), 0, st,
                       p, (int)tiles);
  else
    hipLaunchKernelGGL(lbsa::store_v_chunk_kernel<false>, dim3((unsigned)(B * tiles), num_kv_heads), dim3(256), 0, st,
                       p, (int)tiles);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
