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

// Tuning knobs (compile-time):
//   LBSA_DECODE_KB    32-token k-blocks per loop iteration (1: half a 64-token page, 2: a page)
//   LBSA_DECODE_PIPE  1: double-buffer the K/V registers so the next chunk's loads are in flight
//                     while the current chunk is computed
//   LBSA_DECODE_NT    1: non-temporal hint on the KV stream loads
#ifndef LBSA_DECODE_KB
#define LBSA_DECODE_KB 2
#endif
#ifndef LBSA_DECODE_PIPE
#define LBSA_DECODE_PIPE 1
#endif
#ifndef LBSA_DECODE_NT
#define LBSA_DECODE_NT 0
#endif

constexpr int kKB = LBSA_DECODE_KB;
constexpr int kChunk = 32 * kKB;   // tokens per loop iteration
constexpr int kMinPage = kChunk;   // a chunk never straddles two pages

#if LBSA_DECODE_NT
constexpr int kKvAux = 2;   // buffer-load cache policy: non-temporal
#else
constexpr int kKvAux = 0;
#endif

// K/V registers of one chunk, laid out as MFMA operands.
struct Chunk {
  u32x4 k[kKB][2][4];   // k-block, S-tile, dim block of 32: token row tok0 + 4j, dims 32c + 8grp
  u32x4 v[kKB][8];      // k-block, dim tile of 16: dim 16n + r, tokens 8grp .. 8grp+7
};

struct Lane {
  int r, grp, tok0;
  int k_off;   // byte offset of this lane's K fragment inside a (page, head) block
  int v_off;   // byte offset of this lane's V fragment inside a (page, head) block
};

__device__ __forceinline__ u32x4 buf_load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kKvAux));
}

// One chunk = tokens [off, off + kChunk) of one (page, KV head) block.  Buffer descriptors bound
// each load to its 16 KiB block (a load outside it would return zeros, never fault); the lane's
// offset is one VGPR and the per-load offsets are scalar.
__device__ __forceinline__ void load_chunk(Chunk& ch, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int off,
                                           int page, const Lane& ln) {
#pragma unroll
  for (int kb_i = 0; kb_i < kKB; ++kb_i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        ch.k[kb_i][j][c] = buf_load(kr, ln.k_off + (4 * j * kD + 32 * c) * 2, (off + 32 * kb_i) * kD * 2);
#pragma unroll
  for (int kb_i = 0; kb_i < kKB; ++kb_i)
#pragma unroll
    for (int n = 0; n < 8; ++n) ch.v[kb_i][n] = buf_load(vr, ln.v_off, (16 * n * page + off + 32 * kb_i) * 2);
}

// Online-softmax state of one wave for its 8 query heads (lane: head r; o: dims 16n + 4grp + i).
struct State {
  float m_ref;    // reference max the probabilities are taken against, log2 units
  float m_true;   // true running max, log2 units
  float l;        // this lane's share of sum 2^(s - m_ref)
  f32x4 o[8];
};

constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ void compute_chunk(Chunk& ch, State& st, const u32x4 (&qf)[4], int c0, int kv_begin,
                                              int kv_end, float scale_log2, const Lane& ln) {
  // scores: sc[kb][4j + i] is token c0 + 32kb + 8grp + 4j + i of head r
  float sc[kKB][8];
#pragma unroll
  for (int kb_i = 0; kb_i < kKB; ++kb_i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma16x16x32(ch.k[kb_i][j][c], qf[c], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[kb_i][4 * j + i] = acc[i] * scale_log2;
    }

  if (c0 < kv_begin || c0 + kChunk > kv_end) {
#pragma unroll
    for (int kb_i = 0; kb_i < kKB; ++kb_i) {
      const int t0 = c0 + 32 * kb_i + 8 * ln.grp;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sc[kb_i][e] = (t0 + e < kv_begin || t0 + e >= kv_end) ? -INFINITY : sc[kb_i][e];
      // masked tokens may hold any bits (NaN included), and p = 0 does not cancel a NaN
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 2 * i;
        const uint32_t keep = ((t >= kv_begin && t < kv_end) ? 0x0000ffffu : 0u) |
                              ((t + 1 >= kv_begin && t + 1 < kv_end) ? 0xffff0000u : 0u);
#pragma unroll
        for (int n = 0; n < 8; ++n) ch.v[kb_i][n][i] &= keep;
      }
    }
  }

  float mx = -INFINITY;
#pragma unroll
  for (int kb_i = 0; kb_i < kKB; ++kb_i)
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sc[kb_i][e]);
  mx = fmaxf(mx, xor_lane(mx, 16));
  mx = fmaxf(mx, xor_lane(mx, 32));
  st.m_true = fmaxf(st.m_true, mx);
  // Lazy rescaling: probabilities are taken relative to a reference max that moves only when a
  // score exceeds it by more than kRescaleSlack (log2 units), so p <= 2^kRescaleSlack and the
  // O accumulators are rescaled in rare, wave-uniform steps instead of every chunk.
  const bool need = mx > st.m_ref + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float m_new = need ? mx : st.m_ref;
    const float alpha = fast_exp2(st.m_ref - m_new);   // 1 where unchanged, 0 from -inf
    st.m_ref = m_new;
    st.l *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] *= alpha;
  }
  const float m_use = (st.m_ref == -INFINITY) ? 0.f : st.m_ref;
  float sum = 0.f;
#pragma unroll
  for (int kb_i = 0; kb_i < kKB; ++kb_i) {
    float ps[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ps[e] = fast_exp2(sc[kb_i][e] - m_use);
      sum += ps[e];
    }
    // P split into bf16 hi + lo parts: two MFMAs keep ~16 significant bits of each probability
    u32x4 phi, plo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t hv = pack_bf16(ps[2 * i], ps[2 * i + 1]);
      phi[i] = hv;
      plo[i] = pack_bf16(ps[2 * i] - bf16_lo(hv), ps[2 * i + 1] - bf16_hi(hv));
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      st.o[n] = mfma16x16x32(ch.v[kb_i][n], phi, st.o[n]);
      st.o[n] = mfma16x16x32(ch.v[kb_i][n], plo, st.o[n]);
    }
  }
  st.l += sum;
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void splitkv_decode_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  // wave index is uniform across the wave; say so, so page addressing stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x / p.W;
  const int w = blockIdx.x / G;
  const int h = (blockIdx.x % G) * WAVES + wave;   // KV head of this wave
  Lane ln;
  ln.r = lane & 15;                                 // MFMA row / column index
  ln.grp = lane >> 4;                               // MFMA k group
  // S-tile j row r is token 8*(r/4) + 4j + r%4, so C rows 4grp+i of tile j are tokens 8grp+4j+i
  ln.tok0 = 8 * (ln.r >> 2) + (ln.r & 3);
  ln.k_off = (ln.tok0 * kD + 8 * ln.grp) * 2;
  ln.v_off = (ln.r * p.page + 8 * ln.grp) * 2;
  const int block_bytes = p.page * kD * 2;

  uint64_t t_start = 0;
  if (p.timing && threadIdx.x == 0) t_start = realtime();

  const int U = p.map[7];
  const int32_t* worker_ptr = p.map + 8;
  const int32_t* segs = p.map + 8 + (p.W + 1) + (U + 1) + 2 * U;
  const int s_begin = worker_ptr[w];
  const int s_end = min(worker_ptr[w + 1], p.S);
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
      const uint16_t* qp = p.q + ((size_t)b * p.Hq + h * 8 + (ln.r & 7)) * kD + 8 * ln.grp;
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[c] = ld16(qp + 32 * c);
    }

    State st;
    st.m_ref = -INFINITY;
    st.m_true = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // block-table window: lane i holds the physical page of logical page win + i
    const int32_t* bt_row = p.block_table + (size_t)b * p.bt_stride;
    const int last_page = kv_end > 0 ? (kv_end - 1) / p.page : -1;
    int win = (kv_begin & ~(kChunk - 1)) / p.page;
    int btv = 0;
    auto load_window = [&]() {
      const int lp = win + lane;
      int v = 0;
      if (lp <= last_page) v = bt_row[lp];
      btv = min(max(v, 0), p.num_pages - 1);
    };
    // descriptors of the (page, KV head) blocks holding chunk c, and c's offset in the page;
    // chunks are visited in order, so the page index advances without a division
    int pg_cur = (kv_begin & ~(kChunk - 1)) / p.page;
    int off_cur = (kv_begin & ~(kChunk - 1)) - pg_cur * p.page;
    auto chunk_rsrc = [&](int c, __amdgpu_buffer_rsrc_t& kr, __amdgpu_buffer_rsrc_t& vr) -> int {
      (void)c;
      const int pg = pg_cur;
      const int off = off_cur;
      off_cur += kChunk;
      if (off_cur == p.page) {
        off_cur = 0;
        ++pg_cur;
      }
      if (pg - win >= 64) {
        win = pg;
        load_window();
      }
      const int pid = __builtin_amdgcn_readlane(btv, pg - win);
      const size_t blk = ((size_t)pid * p.Hkv + h) * head_stride;
      kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.k + blk), (short)0, block_bytes, 0x00020000);
      vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.v + blk), (short)0, block_bytes, 0x00020000);
      return off;
    };

    int c = kv_begin & ~(kChunk - 1);
    if (c < kv_end) {
      load_window();
      __amdgpu_buffer_rsrc_t kr, vr;
#if LBSA_DECODE_PIPE
      Chunk A, B;
      int off = chunk_rsrc(c, kr, vr);
      load_chunk(A, kr, vr, off, p.page, ln);
      while (true) {
        int cn = c + kChunk;
        bool more = cn < kv_end;
        if (more) {
          off = chunk_rsrc(cn, kr, vr);
          load_chunk(B, kr, vr, off, p.page, ln);
        }
        compute_chunk(A, st, qf, c, kv_begin, kv_end, p.scale_log2, ln);
        c = cn;
        if (!more) break;
        cn = c + kChunk;
        more = cn < kv_end;
        if (more) {
          off = chunk_rsrc(cn, kr, vr);
          load_chunk(A, kr, vr, off, p.page, ln);
        }
        compute_chunk(B, st, qf, c, kv_begin, kv_end, p.scale_log2, ln);
        c = cn;
        if (!more) break;
      }
#else
      Chunk A;
      for (; c < kv_end; c += kChunk) {
        const int off = chunk_rsrc(c, kr, vr);
        load_chunk(A, kr, vr, off, p.page, ln);
        compute_chunk(A, st, qf, c, kv_begin, kv_end, p.scale_log2, ln);
      }
#endif
    }

    // express the partial against the true max: m = max score, l and o scaled to match
    const float to_true = (st.m_true == -INFINITY) ? 0.f : fast_exp2(st.m_ref - st.m_true);
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] *= to_true;
    float l = st.l * to_true;
    l += xor_lane(l, 16);
    l += xor_lane(l, 32);
    if (ln.r < 8) {
      const size_t row = (size_t)s * p.Hq + h * 8 + ln.r;
      if (ln.grp == 0) {
        p.part_m[row] = (st.m_true == -INFINITY) ? -INFINITY : st.m_true * kLn2;
        p.part_l[row] = l;
      }
      float* dst = p.part_o + row * kD + 4 * ln.grp;
#pragma unroll
      for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4*>(dst + 16 * n) = st.o[n];
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
  if (head_dim != kD || num_q_heads != 8 * num_kv_heads || page_size % kMinPage != 0)
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
