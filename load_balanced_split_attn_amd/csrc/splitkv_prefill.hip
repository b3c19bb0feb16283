// Split-KV chunked prefill over a cached prefix, driven by the same greedy work map.
//
// The pages' load-balanced scheduler ([P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案;
// [P4] "腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级" §二.1) applied to prefill units: a unit
// is a 128-row block of one request's query chunk, cut into 512-token KV tiles that the planner
// packs onto workers exactly as in decode.  Prefix-cache reuse ([P3] §6) means each chunk attends
// to a long cached prefix plus itself under a causal mask: row j of a q_len-row chunk sits at
// position kv_len - q_len + j and sees keys [0, that position].
//
// gfx950 design.  Workgroup = (worker w, KV head g, query head h of the group), 4 waves; wave v
// owns the 32 query rows 32v .. 32v+31 of the unit.  Each 64-key chunk of K (token-major) and V
// (dim-major) is staged once in LDS (double-buffered; global loads for the next chunk are in flight
// while the current one is computed) and read by all four waves: 128 query rows per K/V load, and
// the eight query heads of a KV head run as eight workgroups on one XCD so K/V come from one L2.
// Per wave, with the query rows as the MFMA columns:
//   S^T (keys x rows) = K . Q^T       v_mfma_f32_16x16x32_bf16, Q^T fragments held in VGPRs
//   O^T (dims x rows) += V^T . P^T    same instruction, P as bf16 hi + lo parts
// so every lane holds whole columns: the softmax max/sum of a row needs only in-lane reductions and
// two lane exchanges, exactly as in the decode kernel.  Key tiles are interleaved in 4-key groups so
// that a lane's 8 scores per 32 keys are the 8 consecutive keys it supplies to the PV product.

#include "common.h"
#include "lbsa.h"

namespace lbsa {

struct PrefillParams {
  const uint16_t* q;            // [rows, Hq, 128]
  const uint16_t* k;            // [pages, Hkv, page, 128]
  const uint16_t* v;            // [pages, Hkv, 128, page]
  const int32_t* block_table;   // [B, bt_stride]
  const int32_t* q_lens;        // [B]
  const int32_t* q_start;       // [B]
  const int32_t* kv_lens;       // [B]
  const int32_t* map;
  float* part_m;                // [S, 128, Hq]
  float* part_l;                // [S, 128, Hq]
  float* part_o;                // [S, 128, Hq, 128]
  int32_t bt_stride, num_pages, W, S, B, Hq, Hkv, page, causal;
  float scale_log2;
};

constexpr int kPD = 128;          // head dim
constexpr int kPChunk = 64;       // keys per staged chunk
constexpr int kQTile = 128;       // query rows per unit
constexpr int kColBlocks = 2;     // 16-row column blocks per wave (32 rows)
constexpr int kKRow = kPD * 2;             // LDS bytes per key row of K (16-byte granules XOR-swizzled)
constexpr int kVRow = kPChunk * 2 + 16;    // LDS bytes per dim row of V^T (padded by one granule)
constexpr int kKBytes = kPChunk * kKRow;   // 17408
constexpr int kVBytes = kPD * kVRow;       // 18432
constexpr int kStage = kKBytes + kVBytes;  // one buffer
constexpr float kPRescaleSlack = 8.0f;

__device__ __forceinline__ u32x4 lds_ld16(const uint8_t* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// K rows are 256 B (16 granules).  The 16 lanes of one ds_read_b128 read the same granule of keys
// {0-3, 8-11, 16-19, 24-27} (+4): granule G of key k sits at slot G ^ swz(k), which gives those 16
// keys 16 different bank groups.
__device__ __forceinline__ int k_slot(int key, int granule) {
  const int swz = (key & 3) | (((key >> 3) & 3) << 2);
  return key * kKRow + 16 * (granule ^ swz);
}

__global__ __launch_bounds__(256) void splitkv_prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;
  const int grp = lane >> 4;

  // block -> (worker, KV head, query head of the group); the eight workgroups of one
  // (worker, KV head) land on the same XCD (dispatch is round-robin over 8 XCDs) and are
  // dispatched together, so the K/V they share comes from one L2
  const int f = blockIdx.x;
  const int xcd = f & 7;
  const int kq = f >> 3;
  const int hq = kq & 7;
  const int wg_index = (kq >> 3) * 8 + xcd;      // (w * Hkv + g)
  const int w = wg_index / p.Hkv;
  const int g = wg_index - w * p.Hkv;
  if (w >= p.W) return;
  const int h = g * 8 + hq;                        // query head of this workgroup
  const int rbase = 32 * wave;                     // first row (inside the unit) of this wave

  const int U = p.map[7];
  const int32_t* worker_ptr = p.map + 8;
  const int32_t* segs = p.map + 8 + (p.W + 1) + (U + 1) + 2 * U;
  const int s_begin = worker_ptr[w];
  const int s_end = min(worker_ptr[w + 1], p.S);
  const int block_bytes = p.page * kPD * 2;

  for (int s = s_begin; s < s_end; ++s) {
    const int b = segs[4 * s];
    const int qt = segs[4 * s + 1];
    const int kv_begin = segs[4 * s + 2];
    int kv_end = segs[4 * s + 3];
    if (b < 0 || b >= p.B) continue;
    const int q_len = p.q_lens[b];
    const int kv_len = p.kv_lens[b];
    const int prefix = kv_len - q_len;
    kv_end = min(kv_end, kv_len);
    kv_end = min(kv_end, p.bt_stride * p.page);
    const int unit_row0 = qt * kQTile;                 // first row of the unit inside the chunk
    const int wave_row0 = unit_row0 + rbase;           // first row of this wave
    // last key any row of this wave may see (-1: the wave has no row inside the chunk)
    const int wave_last_key = wave_row0 >= q_len ? -1
                              : (p.causal ? prefix + min(wave_row0 + 32 * kColBlocks - 1, q_len - 1) : kv_len - 1);

    // Q^T fragments: column r of block cb = row wave_row0 + 16cb + r, k = dims 32ks + 8grp .. +7
    u32x4 qf[kColBlocks][4];
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      const int row = wave_row0 + 16 * cb + r;
      const bool ok = row < q_len;
      const uint16_t* qp = p.q + ((size_t)(p.q_start[b] + (ok ? row : 0)) * p.Hq + h) * kPD + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[cb][ks] = ok ? ld16(qp + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
    }

    float m_ref[kColBlocks], m_true[kColBlocks], lsum[kColBlocks];
    f32x4 o[kColBlocks][8];
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      m_ref[cb] = -INFINITY;
      m_true[cb] = -INFINITY;
      lsum[cb] = 0.f;
#pragma unroll
      for (int n = 0; n < 8; ++n) o[cb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t* bt_row = p.block_table + (size_t)b * p.bt_stride;
    const int c_first = kv_begin & ~(kPChunk - 1);
    // chunk staging: every thread loads 4 K granules (key idx/16, dims 8*(idx%16)) and 4 V^T
    // granules (dim idx/8, keys 8*(idx%8)) into registers, computes, then stores them to LDS
    u32x4 kreg[4], vreg[4];
    auto load_chunk = [&](int c) {
      const int pg = c / p.page;
      const int off = c - pg * p.page;
      int pid = bt_row[pg];
      pid = min(max(pid, 0), p.num_pages - 1);
      const size_t blk = ((size_t)pid * p.Hkv + g) * (size_t)p.page * kPD;
      __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.k + blk), (short)0, block_bytes, 0x00020000);
      __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.v + blk), (short)0, block_bytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i;
        kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                kr, ((off + (idx >> 4)) * kPD + 8 * (idx & 15)) * 2, 0, 0));
        vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                vr, ((idx >> 3) * p.page + off + 8 * (idx & 7)) * 2, 0, 0));
      }
    };
    auto store_chunk = [&](int buf_) {
      uint8_t* kd = smem + buf_ * kStage;
      uint8_t* vd = kd + kKBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i;
        *reinterpret_cast<u32x4*>(kd + k_slot(idx >> 4, idx & 15)) = kreg[i];
        *reinterpret_cast<u32x4*>(vd + (idx >> 3) * kVRow + 16 * (idx & 7)) = vreg[i];
      }
    };

    if (c_first < kv_end) {
      load_chunk(c_first);
      store_chunk(0);
    }
    int buf = 0;
    for (int c0 = c_first; c0 < kv_end; c0 += kPChunk, buf ^= 1) {
      __syncthreads();   // chunk c0 is in LDS buffer `buf`; every wave is done with buffer buf^1
      const bool more = c0 + kPChunk < kv_end;
      if (more) load_chunk(c0 + kPChunk);   // in flight while chunk c0 is computed
      if (c0 > wave_last_key) {
        // chunk entirely past this wave's causal diagonal: only help staging
        if (more) store_chunk(buf ^ 1);
        continue;
      }
      // chunk entirely above this wave's causal diagonal: nothing to do (still joins the barriers)
      if (c0 > wave_last_key) continue;
      const uint8_t* kd = smem + buf * kStage;
      const uint8_t* vd = kd + kKBytes;
      // mask needed: keys outside [kv_begin, kv_end), or (causal) keys after some row's position
      const bool edge = (c0 < kv_begin) || (c0 + kPChunk > kv_end) ||
                        (p.causal && c0 + kPChunk - 1 > prefix + wave_row0);

#pragma unroll 1
      for (int kb = 0; kb < 2; ++kb) {
        const int kbase = c0 + 32 * kb;
        // scores: sc[cb][4j+i] = key kbase + 8grp + 4j + i, column (row) r of block cb
        float sc[kColBlocks][8];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * j + (r & 3);
          u32x4 kf[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) kf[ks] = lds_ld16(kd, k_slot(key, 4 * ks + grp));
#pragma unroll
          for (int cb = 0; cb < kColBlocks; ++cb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(kf[ks], qf[cb][ks], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[cb][4 * j + i] = acc[i] * p.scale_log2;
          }
        }
        // V^T fragments of this 32-key block: dim 16n + r, keys kbase + 8grp .. +7
        u32x4 vf[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) vf[n] = lds_ld16(vd, (16 * n + r) * kVRow + (32 * kb + 8 * grp) * 2);
        if (edge) {
#pragma unroll
          for (int cb = 0; cb < kColBlocks; ++cb) {
            const int row = wave_row0 + 16 * cb + r;
            const int last = p.causal ? prefix + row : kv_len - 1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int t = kbase + 8 * grp + e;
              if (t < kv_begin || t >= kv_end || t > last) sc[cb][e] = -INFINITY;
            }
          }
          // keys outside [kv_begin, kv_end) may hold any bits; p = 0 does not cancel a NaN
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = kbase + 8 * grp + 2 * i;
            const uint32_t keep = ((t >= kv_begin && t < kv_end) ? 0x0000ffffu : 0u) |
                                  ((t + 1 >= kv_begin && t + 1 < kv_end) ? 0xffff0000u : 0u);
#pragma unroll
            for (int n = 0; n < 8; ++n) vf[n][i] &= keep;
          }
        }
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb) {
          float mx = sc[cb][0];
#pragma unroll
          for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[cb][e]);
          mx = fmaxf(mx, xor_lane(mx, 16));
          mx = fmaxf(mx, xor_lane(mx, 32));
          m_true[cb] = fmaxf(m_true[cb], mx);
          const bool need = mx > m_ref[cb] + kPRescaleSlack;
          if (__builtin_amdgcn_ballot_w64(need)) {
            const float m_new = need ? mx : m_ref[cb];
            const float alpha = fast_exp2(m_ref[cb] - m_new);
            m_ref[cb] = m_new;
            lsum[cb] *= alpha;
#pragma unroll
            for (int n = 0; n < 8; ++n) o[cb][n] *= alpha;
          }
          const float m_use = (m_ref[cb] == -INFINITY) ? 0.f : m_ref[cb];
          float ps[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            ps[e] = fast_exp2(sc[cb][e] - m_use);
            lsum[cb] += ps[e];
          }
          u32x4 phi, plo;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t hv = pack_bf16(ps[2 * i], ps[2 * i + 1]);
            phi[i] = hv;
            plo[i] = pack_bf16(ps[2 * i] - bf16_lo(hv), ps[2 * i + 1] - bf16_hi(hv));
          }
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            o[cb][n] = mfma16x16x32(vf[n], phi, o[cb][n]);
            o[cb][n] = mfma16x16x32(vf[n], plo, o[cb][n]);
          }
        }
      }
      if (more) store_chunk(buf ^ 1);
    }
    __syncthreads();   // all waves are done with LDS before the next segment stages into it

    // write the partials of this wave's 64 rows (rows past the chunk's end are not stored)
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      const float to_true = (m_true[cb] == -INFINITY) ? 0.f : fast_exp2(m_ref[cb] - m_true[cb]);
      float l = lsum[cb] * to_true;
      l += xor_lane(l, 16);
      l += xor_lane(l, 32);
      const int row_in_unit = rbase + 16 * cb + r;
      if (unit_row0 + row_in_unit < q_len) {
        const size_t slot = ((size_t)s * kQTile + row_in_unit) * p.Hq + h;
        if (grp == 0) {
          p.part_m[slot] = (m_true[cb] == -INFINITY) ? -INFINITY : m_true[cb] * kLn2;
          p.part_l[slot] = l;
        }
        float* dst = p.part_o + slot * kPD + 4 * grp;
#pragma unroll
        for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4*>(dst + 16 * n) = o[cb][n] * to_true;
      }
    }
  }
}

}  // namespace lbsa

using namespace lbsa;

extern "C" int attn_splitkv_prefill(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                                    const int32_t* q_lens, const int32_t* q_start, const int32_t* kv_lens,
                                    const int32_t* map, int32_t num_workers, int32_t num_segments, int32_t B,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                    int32_t q_tile, int32_t causal, float softmax_scale, float* part_m,
                                    float* part_l, float* part_o, void* stream) {
  if (num_workers < 1 || num_segments < 0 || B < 0 || num_kv_heads < 1 || num_pages < 1 ||
      block_table_stride < 0 || page_size < 1)
    return LBSA_ERR_INVALID;
  if (!q || !k_cache || !v_cache || !block_table || !q_lens || !q_start || !kv_lens || !map)
    return LBSA_ERR_INVALID;
  if (num_segments > 0 && (!part_m || !part_l || !part_o)) return LBSA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(part_o)) & 15)
    return LBSA_ERR_INVALID;
  if (head_dim != kPD || num_q_heads != 8 * num_kv_heads || page_size % kPChunk != 0 || q_tile != kQTile)
    return LBSA_ERR_UNSUPPORTED;
  PrefillParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.block_table = block_table;
  p.q_lens = q_lens;
  p.q_start = q_start;
  p.kv_lens = kv_lens;
  p.map = map;
  p.part_m = part_m;
  p.part_l = part_l;
  p.part_o = part_o;
  p.bt_stride = block_table_stride;
  p.num_pages = num_pages;
  p.W = num_workers;
  p.S = num_segments;
  p.B = B;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.page = page_size;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = softmax_scale * kLog2e;
  // (worker, KV head) pairs padded to a multiple of 8, times the 8 query heads of a group
  const int64_t pairs = (int64_t)num_workers * num_kv_heads;
  const int64_t grid = ((pairs + 7) / 8) * 8 * 8;
  if (grid > INT32_MAX) return LBSA_ERR_INVALID;
  hipLaunchKernelGGL(splitkv_prefill_kernel, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     p);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
