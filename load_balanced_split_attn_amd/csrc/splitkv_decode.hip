// Split-KV decode attention over a paged bf16 KV cache, driven by a precomputed work map.
//
// Method: [P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案 step 4 and [P4]
// "腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级" §二.1: every worker reads its own list
// from the global task map and computes split-KV partial results for it.  GQA shape of [P3] §2
// (8 query heads per KV head, head dim 128).
//
// gfx950 design.  A workgroup is (worker w, KV-head group g) with one 64-lane wave per KV head
// of the group; waves are independent (no LDS, no barriers).  For each segment (b, kv_begin,
// kv_end) of list w a wave streams the segment's KV in 32-token chunks:
//
//   * K chunk (32 tokens x 128 dims, token-major in the page) and V chunk (128 dims x 32 tokens,
//     dim-major in the page) go straight from HBM into VGPRs with 16-byte loads laid out as MFMA
//     operands, so no LDS round trip is needed;
//   * S = K . Q^T with v_mfma_f32_16x16x32_bf16: rows are tokens, columns are the 8 query heads
//     of the KV head (columns 8..15 repeat them and are ignored);  the two 16-token row tiles are
//     interleaved so each lane ends up holding the scores of 8 consecutive tokens of one head,
//     exactly the k-slice it must supply to the PV product;
//   * online softmax in the exp2 domain per lane (head = lane % 16), the chunk maximum reduced
//     across the four 16-lane groups with two lane exchanges;
//   * O^T += V^T . P^T with the same MFMA; P is split into bf16 hi + lo parts (two MFMAs) so the
//     probabilities keep ~16 significant bits and the product stays within fp32-accumulate
//     accuracy;
//   * at segment end the wave writes (m, l, o) for its 8 query heads to partial slot = segment id.
//
// The contractions are tiny (8 query heads) and the kernel is HBM-bound: MFMA work per chunk is
// ~24 instructions against 16 KiB of loads.  The matrix cores take the dot products off the VALU,
// whose fp32 FMA budget at full HBM rate would otherwise be nearly exhausted (about 2,300 VALU
// lane operations per token and KV head for QK, PV and softmax, against ~2,500 available).

#include "common.h"
#include "lbsa.h"

namespace lbsa {

struct DecodeParams {
  const uint16_t* q;            // [B, Hq, 128]
  const uint16_t* k;            // [pages, Hkv, page, 128]
  const uint16_t* v;            // [pages, Hkv, 128, page]
  const int32_t* block_table;   // [B, bt_stride]
  const int32_t* seq_lens;      // [B]
  const int32_t* map;
  float* part_m;                // [S, Hq]
  float* part_l;                // [S, Hq]
  float* part_o;                // [S, Hq, 128]
  uint64_t* timing;             // [grid, 4] or null
  int32_t bt_stride, num_pages, W, S, B, Hq, Hkv, page;
  float scale_log2;             // softmax scale * log2(e)
};

constexpr int kD = 128;
constexpr int kChunk = 32;

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void splitkv_decode_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = gridDim.x / p.W;
  const int w = blockIdx.x / G;
  const int h = (blockIdx.x % G) * WAVES + wave;   // KV head of this wave
  const int r = lane & 15;                          // MFMA row / column index
  const int grp = lane >> 4;                        // MFMA k group

  uint64_t t_start = 0;
  if (p.timing && threadIdx.x == 0) t_start = realtime();

  const int U = p.map[7];
  const int32_t* worker_ptr = p.map + 8;
  const int32_t* segs = p.map + 8 + (p.W + 1) + (U + 1) + 2 * U;
  const int s_begin = worker_ptr[w];
  const int s_end = min(worker_ptr[w + 1], p.S);

  // token row of S-tile j held by lane row r: tiles interleave 4-token groups so that C rows
  // 4*grp+i of tile j are tokens 8*grp + 4*j + i
  const int tok0 = 8 * (r >> 2) + (r & 3);
  const size_t head_stride = (size_t)p.page * kD;   // elements per (page, KV head) block

  for (int s = s_begin; s < s_end; ++s) {
    const int b = segs[4 * s];
    const int kv_begin = segs[4 * s + 2];
    int kv_end = segs[4 * s + 3];
    if (b < 0 || b >= p.B) continue;
    kv_end = min(kv_end, p.seq_lens[b]);
    kv_end = min(kv_end, p.bt_stride * p.page);

    // Q^T fragments: column r = query head 8h + (r & 7), k = dims 32c + 8grp .. +7
    u32x4 qf[4];
    {
      const uint16_t* qp = p.q + ((size_t)b * p.Hq + h * 8 + (r & 7)) * kD + 8 * grp;
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[c] = ld16(qp + 32 * c);
    }

    float m = -INFINITY;   // running max (log2 units) of head r
    float l = 0.f;         // this lane's share of the running sum
    f32x4 o[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = kv_begin & ~(kChunk - 1); c0 < kv_end; c0 += kChunk) {
      const int pg = c0 / p.page;
      const int off = c0 - pg * p.page;
      int pid = p.block_table[(size_t)b * p.bt_stride + pg];
      pid = min(max(pid, 0), p.num_pages - 1);
      const uint16_t* kb = p.k + ((size_t)pid * p.Hkv + h) * head_stride + (size_t)off * kD;
      const uint16_t* vb = p.v + ((size_t)pid * p.Hkv + h) * head_stride + off;

      u32x4 kr[2][4];
      u32x4 vr[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) kr[j][c] = ld16(kb + (size_t)(tok0 + 4 * j) * kD + 32 * c + 8 * grp);
#pragma unroll
      for (int n = 0; n < 8; ++n) vr[n] = ld16(vb + (size_t)(16 * n + r) * p.page + 8 * grp);

      f32x4 sacc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) sacc[j] = mfma16x16x32(kr[j][c], qf[c], sacc[j]);
      }

      // sc[4j + i] is the score of token c0 + 8grp + 4j + i for head r
      float sc[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[4 * j + i] = sacc[j][i] * p.scale_log2;

      const bool partial = (c0 < kv_begin) || (c0 + kChunk > kv_end);
      if (partial) {
        uint32_t keep[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = c0 + 8 * grp + e;
          if (t < kv_begin || t >= kv_end) sc[e] = -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = c0 + 8 * grp + 2 * i;
          keep[i] = ((t >= kv_begin && t < kv_end) ? 0x0000ffffu : 0u) |
                    ((t + 1 >= kv_begin && t + 1 < kv_end) ? 0xffff0000u : 0u);
        }
        // masked tokens may hold any bits (NaN included) and p = 0 does not cancel NaN
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) vr[n][i] &= keep[i];
      }

      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, xor_lane(mx, 16));
      mx = fmaxf(mx, xor_lane(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_ref);
      m = m_new;

      float ps[8];
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ps[e] = fast_exp2(sc[e] - m_ref);
        sum += ps[e];
      }
      l = l * alpha + sum;

      u32x4 phi, plo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t hv = pack_bf16(ps[2 * i], ps[2 * i + 1]);
        phi[i] = hv;
        plo[i] = pack_bf16(ps[2 * i] - bf16_lo(hv), ps[2 * i + 1] - bf16_hi(hv));
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        o[n] *= alpha;
        o[n] = mfma16x16x32(vr[n], phi, o[n]);
        o[n] = mfma16x16x32(vr[n], plo, o[n]);
      }
    }

    l += xor_lane(l, 16);
    l += xor_lane(l, 32);
    if (r < 8) {
      const size_t row = (size_t)s * p.Hq + h * 8 + r;
      if (grp == 0) {
        p.part_m[row] = (m == -INFINITY) ? -INFINITY : m * kLn2;
        p.part_l[row] = l;
      }
      float* dst = p.part_o + row * kD + 4 * grp;
#pragma unroll
      for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4*>(dst + 16 * n) = o[n];
    }
  }

  if (p.timing) {
    if constexpr (WAVES > 1) __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t* rec = p.timing + 4 * (size_t)blockIdx.x;
      rec[0] = t_start;
      rec[1] = realtime();
      rec[2] = hw_id();
      rec[3] = xcc_id();
    }
  }
}

template <int WAVES>
hipError_t launch_decode(const DecodeParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(splitkv_decode_kernel<WAVES>, dim3(grid), dim3(64 * WAVES), 0, stream, p);
  return hipGetLastError();
}

template <int WAVES>
int decode_blocks_per_cu() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, splitkv_decode_kernel<WAVES>, 64 * WAVES, 0) !=
      hipSuccess)
    return 0;
  return nb;
}

}  // namespace lbsa

using namespace lbsa;

extern "C" int attn_splitkv(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                            const int32_t* seq_lens, const int32_t* map, int32_t num_workers,
                            int32_t num_segments, int32_t head_groups, int32_t B, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            float softmax_scale, float* part_m, float* part_l, float* part_o,
                            uint64_t* timing, void* stream) {
  if (num_workers < 1 || num_segments < 0 || B < 0 || head_groups < 1 || num_kv_heads < 1 ||
      num_pages < 1 || block_table_stride < 0 || page_size < 1)
    return LBSA_ERR_INVALID;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !map) return LBSA_ERR_INVALID;
  if (num_segments > 0 && (!part_m || !part_l || !part_o)) return LBSA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(part_o)) & 15)
    return LBSA_ERR_INVALID;
  if (head_dim != kD || num_q_heads != 8 * num_kv_heads || page_size % kChunk != 0)
    return LBSA_ERR_UNSUPPORTED;
  if (num_kv_heads % head_groups) return LBSA_ERR_INVALID;
  const int waves = num_kv_heads / head_groups;
  if (waves != 1 && waves != 2 && waves != 4 && waves != 8) return LBSA_ERR_UNSUPPORTED;

  DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.map = map;
  p.part_m = part_m;
  p.part_l = part_l;
  p.part_o = part_o;
  p.timing = timing;
  p.bt_stride = block_table_stride;
  p.num_pages = num_pages;
  p.W = num_workers;
  p.S = num_segments;
  p.B = B;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.page = page_size;
  p.scale_log2 = softmax_scale * kLog2e;

  const int64_t grid = (int64_t)num_workers * head_groups;
  if (grid > INT32_MAX) return LBSA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (waves) {
    case 1: err = launch_decode<1>(p, (int)grid, st); break;
    case 2: err = launch_decode<2>(p, (int)grid, st); break;
    case 4: err = launch_decode<4>(p, (int)grid, st); break;
    default: err = launch_decode<8>(p, (int)grid, st); break;
  }
  return err == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}

extern "C" int attn_query_workers(int device, int32_t head_groups, int32_t* num_workers_out) {
  static int cached[64][9];
  if (!num_workers_out || head_groups < 1 || head_groups > 8 || (8 % head_groups) || device < 0 ||
      device >= 64)
    return LBSA_ERR_INVALID;
  if (cached[device][head_groups] > 0) {
    *num_workers_out = cached[device][head_groups];
    return LBSA_OK;
  }
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return LBSA_ERR_HIP;
  if (hipSetDevice(device) != hipSuccess) return LBSA_ERR_HIP;
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  const int waves = 8 / head_groups;
  int nb = 0;
  if (e == hipSuccess) {
    switch (waves) {
      case 1: nb = decode_blocks_per_cu<1>(); break;
      case 2: nb = decode_blocks_per_cu<2>(); break;
      case 4: nb = decode_blocks_per_cu<4>(); break;
      default: nb = decode_blocks_per_cu<8>(); break;
    }
  }
  hipSetDevice(prev);
  if (e != hipSuccess || nb < 1 || cus < 1) return LBSA_ERR_HIP;
  const int w = cus * nb / head_groups;
  cached[device][head_groups] = w;
  *num_workers_out = w;
  return LBSA_OK;
}
