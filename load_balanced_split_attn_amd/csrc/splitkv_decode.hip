// Split-KV decode attention over a paged KV cache (bf16, or 8-bit E4M3 with per-head scales),
// driven by a precomputed work map.
//
// Method: [P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案 step 4 and [P4]
// "腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级" §二.1: every worker reads its own list
// from the global task map and computes split-KV partial results for it.  GQA shape of [P3] §2
// (8 query heads per KV head, head dim 128).  The 8-bit cache is the production precision of
// [P3] §1 / §14 ("W8A8C8") and §8 (attention in FP8).
//
// gfx950 design.  A workgroup is (worker w, KV-head group g) with one 64-lane wave per KV head
// of the group; waves are independent (no LDS, no barriers).  For each segment (b, kv_begin,
// kv_end) of list w a wave streams the segment's KV in 64-token chunks (one page of 64 tokens, or
// a 64-token slice of a larger page):
//
//   * K chunk (64 tokens x 128 dims) and V chunk (128 dims x 64 tokens) go straight from HBM into
//     VGPRs with 16-byte non-temporal buffer loads laid out as MFMA operands, so no LDS round trip
//     is needed; the cache's blocked layout (below) makes every load instruction read whole
//     128-byte lines; the next chunk's loads are in flight while the current one is computed;
//   * S = K . Q^T with v_mfma_f32_16x16x32_bf16: rows are tokens, columns are the 8 query heads
//     of the KV head (columns 8..15 repeat them and are ignored).  Token rows are assigned so that
//     each lane ends up holding the scores of 8 consecutive tokens of one head, exactly the
//     k-slice it must supply to the PV product;
//   * online softmax in the exp2 domain per lane (head = lane % 16), the chunk maximum reduced
//     across the four 16-lane groups with two lane exchanges;
//   * O^T += V^T . P^T with the same MFMA; P is split into bf16 hi + lo parts (two MFMAs) so the
//     probabilities keep ~16 significant bits and the product stays within fp32-accumulate
//     accuracy;
//   * at segment end the wave writes (m, l, o) for its 8 query heads to partial slot = segment id.
//
// 8-bit cache: the E4M3 codes are widened to bf16 in registers right before the MFMAs
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1, exact: every E4M3 value is a bf16 value); the K scale
// of the head is folded into the softmax scale and the V scale into the partial's o at segment end,
// so the arithmetic on the codes is the bf16 path's.  A chunk is half the bytes of a bf16 chunk;
// its compute is the same plus 128 conversions per lane, still well inside the HBM time of a chunk.
//
// The contractions are tiny (8 query heads) and the kernel is HBM-bound: MFMA work per chunk is
// ~48 instructions against 32 KiB (bf16) or 16 KiB (8-bit) of loads.  The matrix cores take the
// dot products off the VALU, whose fp32 FMA budget at full HBM rate would otherwise be nearly
// exhausted (about 2,300 VALU lane operations per token and KV head for QK, PV and softmax, against
// ~2,500 available at the bf16 byte rate and half that at the 8-bit rate).

#include <atomic>

#include "common.h"
#include "lbsa.h"

namespace lbsa {

struct DecodeParams {
  const uint16_t* q;            // [B, Hq, 128] bf16
  const uint8_t* k;             // [pages, Hkv, page, 128] elements of the cache type
  const uint8_t* v;             // [pages, Hkv, 128, page]
  const float* k_scale;         // [Hkv] for the 8-bit cache, else null
  const float* v_scale;         // [Hkv] for the 8-bit cache, else null
  const int32_t* block_table;   // [B, bt_stride]
  const int32_t* seq_lens;      // [B]
  const int32_t* map;
  float* part_m;                // [S, Hq]
  float* part_l;                // [S, Hq]
  float* part_o;                // [S, Hq, 128]; multi-token decode: [S, R, Hq(, 128)]
  const int32_t* q_lens;        // multi-token decode: [B] query rows of request b (else null)
  const int32_t* q_start;       // multi-token decode: [B] first row of request b in q (else null)
  uint64_t* timing;             // [grid, 4] or null
  int32_t* claim;               // run-time claiming: device int32[2] (next item, workgroups done), else null
  int32_t bt_stride, num_pages, W, S, B, Hq, Hkv, page;
  int32_t G;                    // KV-head groups per list (workgroups per list in the static launch)
  int32_t R;                    // partial rows per slot (1 for plain decode)
  float scale_log2;             // softmax scale * log2(e)
};

constexpr int kD = 128;
constexpr int kRow = 64;           // bytes per row of the blocked cache layout
constexpr int kKB = 2;             // 32-token k-blocks per chunk
constexpr int kChunk = 32 * kKB;   // tokens per chunk
constexpr int kMinPage = kChunk;   // a chunk never straddles two pages


struct Lane {
  int r, grp;
  int k_off;   // byte offset of this lane's K fragment inside a (page, head) block
  int v_off;   // byte offset of this lane's V fragment inside a (page, head) block
};

// KV stream load policy (buffer-load cache-policy bits): 2 = non-temporal (nt), 0 = default.  The
// KV stream is read once; with whole 128-byte lines per load instruction (the blocked cache layout)
// the non-temporal policy streams ~10% faster than the default on gfx950.
#ifndef LBSA_DECODE_KV_POLICY
#define LBSA_DECODE_KV_POLICY 2
#endif
#ifndef LBSA_FP8_KV_POLICY
#define LBSA_FP8_KV_POLICY 2
#endif


template <int POLICY>
__device__ __forceinline__ u32x4 buf_load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, POLICY));
}

// ---- cache element types --------------------------------------------------------------------
//
// Blocked cache layout.  A (page, KV head) block of page_size tokens x 128 dims is stored in rows
// of 64 bytes: K as [128 e / 64 dim tiles][page tokens][64 B] (each row = one token's dims of one
// tile), V as [page e / 64 token tiles][128 dims][64 B] (each row = one dim's tokens of one tile),
// e = element bytes.  Every load instruction below then reads whole 128-byte lines (4 runs of 4
// consecutive K rows, or 16 consecutive V rows), which is what lets the stream run at the
// non-temporal rate.
//
// A type fixes how a lane's 16-byte loads map onto the MFMA operands.  For k-block kb (32 tokens)
// S-tile j (16 token rows) the lane supplies A-row r = one token and, for the four MFMAs c = 0..3
// over the 128 dims, eight dims each; the Q^T fragments use the same dims.  C rows 4grp + i of the
// tile land in lane (r, grp), so the lane's eight scores per k-block are the tokens
// first_token(kb) + e, e = 0..7, and its V operand of that k-block must hold the same tokens.

// bf16 cache (32 elements per 64-byte row): K row r of S-tile (kb, j) is token
// 32kb + 8(r/4) + 4j + r%4; MFMA c takes dims 32c + 8grp .. +7 (dim tile c); V fragment = 8
// consecutive tokens (16 bytes) of dim 16n + r.
struct KvBf16 {
  static constexpr int kElem = 2;
  // loop shape: issue the next chunk only when one exists.  Issuing one per computed chunk (an
  // empty one past the end) measured the same for one query row but needs more registers: the
  // four-row kernel then spills
  static constexpr bool kIssuePastEnd = false;
  static constexpr int kPolicy = LBSA_DECODE_KV_POLICY;
  struct Chunk {
    u32x4 k[kKB][2][4];   // k-block, S-tile, MFMA c
    u32x4 v[kKB][8];      // k-block, dim tile n: dim 16n + r, tokens first_token(kb) .. +7
  };
  __device__ static int first_token(int kb, const Lane& ln) { return 32 * kb + 8 * ln.grp; }
  __device__ static int q_dim(int c, const Lane& ln) { return 32 * c + 8 * ln.grp; }
  __device__ static void setup(Lane& ln) {
    const int tok0 = 8 * (ln.r >> 2) + (ln.r & 3);
    ln.k_off = tok0 * kRow + 16 * ln.grp;
    ln.v_off = ln.r * kRow + 16 * ln.grp;
  }
  __device__ static void load(Chunk& ch, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int off, int page,
                              const Lane& ln) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          ch.k[kb][j][c] = buf_load<kPolicy>(kr, ln.k_off, (c * page + off + 32 * kb + 4 * j) * kRow);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int n = 0; n < 8; ++n)
        ch.v[kb][n] = buf_load<kPolicy>(vr, ln.v_off, ((off / 32 + kb) * kD + 16 * n) * kRow);
  }
  __device__ static u32x4 k_op(const Chunk& ch, int kb, int j, int c) { return ch.k[kb][j][c]; }
  __device__ static u32x4 v_op(const Chunk& ch, int kb, int n) { return ch.v[kb][n]; }
  // zero the V elements of tokens first_token(kb) + 2i (lo) and + 2i + 1 (hi) that are not kept
  __device__ static void mask_v(Chunk& ch, int kb, int i, bool keep_lo, bool keep_hi) {
    const uint32_t keep = (keep_lo ? 0x0000ffffu : 0u) | (keep_hi ? 0xffff0000u : 0u);
#pragma unroll
    for (int n = 0; n < 8; ++n) ch.v[kb][n][i] &= keep;
  }
};

// Two E4M3 codes (bytes 2*hi, 2*hi + 1 of x) -> two bf16 values in one dword, exactly.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
}

// 8-bit (E4M3) cache (64 elements per 64-byte row): K row r of S-tile (kb, j) is token
// 16(r/4) + 8kb + 4j + r%4; the lane's two 16-byte K loads are dims 64h + 16grp .. +15 (dim tile
// h), and MFMA c takes dims 64(c/2) + 16grp + 8(c%2) .. +7; V fragment = 16 consecutive tokens
// (16 bytes) of dim 16n + r, the low 8 for k-block 0 and the high 8 for 1.
struct KvFp8 {
  static constexpr int kElem = 1;
  // loop shape: issue one chunk per computed chunk (an empty one past the end), so the compiler's
  // wait counts stay exact; 1-4% faster than issuing only when a next chunk exists
  static constexpr bool kIssuePastEnd = true;
  static constexpr int kPolicy = LBSA_FP8_KV_POLICY;
  struct Chunk {
    u32x4 k[kKB][2][2];   // k-block, S-tile, dim tile h: dims 64h + 16grp .. +15
    u32x4 v[8];           // dim tile n: dim 16n + r, tokens 16grp .. +15
  };
  __device__ static int first_token(int kb, const Lane& ln) { return 16 * ln.grp + 8 * kb; }
  __device__ static int q_dim(int c, const Lane& ln) { return 64 * (c >> 1) + 16 * ln.grp + 8 * (c & 1); }
  __device__ static void setup(Lane& ln) {
    const int tok0 = 16 * (ln.r >> 2) + (ln.r & 3);
    ln.k_off = tok0 * kRow + 16 * ln.grp;
    ln.v_off = ln.r * kRow + 16 * ln.grp;
  }
  __device__ static void load(Chunk& ch, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int off, int page,
                              const Lane& ln) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          ch.k[kb][j][h] = buf_load<kPolicy>(kr, ln.k_off, (h * page + off + 8 * kb + 4 * j) * kRow);
#pragma unroll
    for (int n = 0; n < 8; ++n) ch.v[n] = buf_load<kPolicy>(vr, ln.v_off, ((off / 64) * kD + 16 * n) * kRow);
  }
  __device__ static u32x4 widen(uint32_t d0, uint32_t d1) {
    return u32x4{e4m3x2_to_bf16x2<false>(d0), e4m3x2_to_bf16x2<true>(d0), e4m3x2_to_bf16x2<false>(d1),
                 e4m3x2_to_bf16x2<true>(d1)};
  }
  __device__ static u32x4 k_op(const Chunk& ch, int kb, int j, int c) {
    const u32x4 raw = ch.k[kb][j][c >> 1];
    return widen(raw[2 * (c & 1)], raw[2 * (c & 1) + 1]);
  }
  __device__ static u32x4 v_op(const Chunk& ch, int kb, int n) { return widen(ch.v[n][2 * kb], ch.v[n][2 * kb + 1]); }
  __device__ static void mask_v(Chunk& ch, int kb, int i, bool keep_lo, bool keep_hi) {
    const int sh = 16 * (i & 1);
    const uint32_t keep = (((keep_lo ? 0x00ffu : 0u) | (keep_hi ? 0xff00u : 0u)) << sh) | ~(0xffffu << sh);
#pragma unroll
    for (int n = 0; n < 8; ++n) ch.v[n][2 * kb + (i >> 1)] &= keep;
  }
};

// ---- online softmax and the PV product ------------------------------------------------------

// Online-softmax state of one wave for one 16-column block (lane: column r; o: dims 16n + 4grp + i).
// Column r of block cb is query head 8h + (r & 7) of query row 2cb + (r >> 3); plain decode has one
// row, so its columns 8..15 repeat the heads and are not stored.
struct State {
  float m_ref;    // reference max the probabilities are taken against, log2 units
  float m_true;   // true running max, log2 units
  float l;        // this lane's share of sum 2^(s - m_ref)
  f32x4 o[8];
};

constexpr float kRescaleSlack = 8.0f;

// One 64-token chunk for NQB column blocks.  Keys outside [kv_begin, kv_end) are masked for every
// column; a column also masks keys at or past vis_end[cb] (the causal end of its query row).
// edge_end is the smallest visible end of any stored row: chunks that end before it and start at or
// after kv_begin need no mask at all.
template <class KV, int NQB>
__device__ __forceinline__ void compute_chunk(typename KV::Chunk& ch, State (&st)[NQB], const u32x4 (&qf)[NQB][4],
                                              int c0, int kv_begin, int kv_end, const int (&vis_end)[NQB],
                                              int edge_end, float scale_log2, const Lane& ln) {
  // scores: sc[cb][kb][4j + i] is token c0 + first_token(kb) + 4j + i of column r of block cb
  float sc[NQB][kKB][8];
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 acc[NQB];
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 kop = KV::k_op(ch, kb, j, c);
#pragma unroll
        for (int cb = 0; cb < NQB; ++cb) acc[cb] = mfma16x16x32(kop, qf[cb][c], acc[cb]);
      }
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[cb][kb][4 * j + i] = acc[cb][i] * scale_log2;
    }

  if (c0 < kv_begin || c0 + kChunk > edge_end) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const int t0 = c0 + KV::first_token(kb, ln);
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sc[cb][kb][e] = (t0 + e < kv_begin || t0 + e >= vis_end[cb]) ? -INFINITY : sc[cb][kb][e];
      // masked tokens may hold any bits (NaN included), and p = 0 does not cancel a NaN
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 2 * i;
        KV::mask_v(ch, kb, i, t >= kv_begin && t < kv_end, t + 1 >= kv_begin && t + 1 < kv_end);
      }
    }
  }

  float m_use[NQB];
#pragma unroll
  for (int cb = 0; cb < NQB; ++cb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sc[cb][kb][e]);
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    st[cb].m_true = fmaxf(st[cb].m_true, mx);
    // Lazy rescaling: probabilities are taken relative to a reference max that moves only when a
    // score exceeds it by more than kRescaleSlack (log2 units), so p <= 2^kRescaleSlack and the
    // O accumulators are rescaled in rare, wave-uniform steps instead of every chunk.
    const bool need = mx > st[cb].m_ref + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      // only columns whose reference moves are rescaled (0 from -inf); the others keep theirs, which
      // may still be -inf for a column with no visible key yet (-inf - -inf would be NaN)
      const float m_new = need ? mx : st[cb].m_ref;
      const float alpha = need ? fast_exp2(st[cb].m_ref - m_new) : 1.f;
      st[cb].m_ref = m_new;
      st[cb].l *= alpha;
#pragma unroll
      for (int n = 0; n < 8; ++n) st[cb].o[n] *= alpha;
    }
    m_use[cb] = (st[cb].m_ref == -INFINITY) ? 0.f : st[cb].m_ref;
  }
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) {
    // P split into bf16 hi + lo parts: two MFMAs keep ~16 significant bits of each probability
    u32x4 phi[NQB], plo[NQB];
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) {
      float ps[8];
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ps[e] = fast_exp2(sc[cb][kb][e] - m_use[cb]);
        sum += ps[e];
      }
      st[cb].l += sum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t hv = pack_bf16(ps[2 * i], ps[2 * i + 1]);
        phi[cb][i] = hv;
        plo[cb][i] = pack_bf16(ps[2 * i] - bf16_lo(hv), ps[2 * i + 1] - bf16_hi(hv));
      }
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const u32x4 vop = KV::v_op(ch, kb, n);
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb) {
        st[cb].o[n] = mfma16x16x32(vop, phi[cb], st[cb].o[n]);
        st[cb].o[n] = mfma16x16x32(vop, plo[cb], st[cb].o[n]);
      }
    }
  }
}

// ---- the kernel -----------------------------------------------------------------------------

// ROWS = 1: plain decode (one query row per request, row b of q, partial rows R = 1).  ROWS = 2 or 4:
// up to ROWS query rows per request (multi-token decode): request b's q_lens[b] rows start at row
// q_start[b] of q and are the last q_lens[b] positions of its context, row j seeing keys
// [0, kv_len - q_len + j]; the map comes from attn_plan_prefill with q_tile = R >= q_lens[b], and
// the partials have R rows per slot.
//
// CLAIM = false: workgroup (w, g) of a W x G grid walks list w for head group g.  CLAIM = true (one
// wave per workgroup): a grid of resident workgroups runs items (list w, KV head g) = (i / G, i % G),
// workgroup b item b first and then, one at a time, the next item from a device counter until
// none is left; every item is run exactly once and writes the same partial slots as in the static
// launch, so the results are bitwise those of the static launch.  The last workgroup to finish
// puts the counter state back to zero.
template <class KV, int WAVES, int ROWS, bool CLAIM = false>
__global__ __launch_bounds__(64 * WAVES) void splitkv_decode_kernel(DecodeParams p) {
  using Chunk = typename KV::Chunk;
  constexpr int NQB = ROWS <= 2 ? 1 : 2;   // 16-column blocks: 8 heads x 2 rows each
  static_assert(!CLAIM || WAVES == 1, "run-time claiming runs one wave per workgroup");
  const int lane = threadIdx.x & 63;
  // wave index is uniform across the wave; say so, so page addressing stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = p.G;
  Lane ln;
  ln.r = lane & 15;                                 // MFMA row / column index
  ln.grp = lane >> 4;                               // MFMA k group
  KV::setup(ln);
  const int block_bytes = p.page * kD * KV::kElem;

  uint64_t t_start = 0;
  if (p.timing && threadIdx.x == 0) t_start = realtime();

  const int version = p.map[0];
  // a device-built map that reported an error, or an unknown layout
  if (version != LBSA_MAP_VERSION && version != LBSA_MAP_VERSION_ORDERED && version != LBSA_MAP_VERSION_PLACED) return;
  // a map planned for another worker count (its lists would be read past their end)
  if (p.map[2] != p.W) return;
  const int U = p.map[7];
  const int32_t* worker_ptr = p.map + 8;
  const int32_t* segs = p.map + 8 + (p.W + 1) + (U + 1) + 2 * U;
  // version 2: worker w runs the segments order[worker_ptr[w] ..), by slot index
  const int32_t* order = version == LBSA_MAP_VERSION_ORDERED ? segs + 4 * p.map[4] : nullptr;
  const size_t head_bytes = (size_t)block_bytes;   // bytes per (page, KV head) block

  // list w for KV head h (this wave)
  auto run_list = [&](int w, int h) __attribute__((always_inline)) {
  const float s_log2 = p.k_scale ? p.scale_log2 * p.k_scale[h] : p.scale_log2;
  const float o_scale = p.v_scale ? p.v_scale[h] : 1.f;
  const int s_begin = worker_ptr[w];
  const int s_end = min(worker_ptr[w + 1], p.S);
  for (int j = s_begin; j < s_end; ++j) {
    const int s = order ? order[j] : j;
    if (s < 0 || s >= p.S) continue;
    const int b = segs[4 * s];
    const int kv_begin = max(segs[4 * s + 2], 0);
    int kv_end = segs[4 * s + 3];
    if (b < 0 || b >= p.B) continue;
    if (ROWS > 1 && segs[4 * s + 1] != 0) continue;   // every request is one unit of R rows
    const int kv_len = p.seq_lens[b];
    kv_end = min(kv_end, kv_len);
    kv_end = min(kv_end, p.bt_stride * p.page);
    const int q_len = ROWS > 1 ? min(p.q_lens[b], p.R) : 1;
    if (q_len <= 0) continue;
    const int q_row0 = ROWS > 1 ? p.q_start[b] : b;

    // Q^T fragments: column r of block cb = query head 8h + (r & 7) of row 2cb + (r >> 3) (zero for
    // rows past q_len), k = dims q_dim(c) .. +7; vis_end = the column's causal key end
    u32x4 qf[NQB][4];
    int vis_end[NQB];
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) {
      const int row = ROWS > 1 ? 2 * cb + (ln.r >> 3) : 0;
      const bool ok = row < q_len;
      const uint16_t* qp = p.q + ((size_t)(q_row0 + (ok ? row : 0)) * p.Hq + h * 8 + (ln.r & 7)) * kD;
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[cb][c] = ok ? ld16(qp + KV::q_dim(c, ln)) : u32x4{0u, 0u, 0u, 0u};
      vis_end[cb] = ok ? min(kv_end, kv_len - q_len + row + 1) : kv_end;
    }
    const int edge_end = ROWS > 1 ? min(kv_end, kv_len - q_len + 1) : kv_end;

    State st[NQB];
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) {
      st[cb].m_ref = -INFINITY;
      st[cb].m_true = -INFINITY;
      st[cb].l = 0.f;
#pragma unroll
      for (int n = 0; n < 8; ++n) st[cb].o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

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
    // chunks are issued in order, so the page index advances without a division
    int c = kv_begin & ~(kChunk - 1);
    int pg_cur = c / p.page;
    int off_cur = c - pg_cur * p.page;
    // Issue the loads of the next chunk into ch.  The buffer descriptors bound each load to its
    // (page, KV head) block (a load outside it returns zeros, never faults); a chunk that is not
    // live (past the segment's end) gets an empty descriptor, so its loads return zeros without
    // touching memory.
    auto issue = [&](Chunk& ch, bool live) {
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
      const size_t blk = ((size_t)pid * p.Hkv + h) * head_bytes;
      const int nbytes = live ? block_bytes : 0;
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.k + blk), (short)0, nbytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.v + blk), (short)0, nbytes, 0x00020000);
      KV::load(ch, kr, vr, off, p.page, ln);
    };

    if (c < kv_end) {
      load_window();
      // double buffer: the next chunk's loads are in flight while the current chunk is computed
      Chunk A, B;
      issue(A, true);
      if constexpr (KV::kIssuePastEnd) {
        // one chunk issued per chunk computed, with no branch around the issue (the last one is
        // empty), so the compiler's wait counts stay exact through the loop
        while (true) {
          issue(B, c + kChunk < kv_end);
          compute_chunk<KV, NQB>(A, st, qf, c, kv_begin, kv_end, vis_end, edge_end, s_log2, ln);
          c += kChunk;
          if (c >= kv_end) break;
          issue(A, c + kChunk < kv_end);
          compute_chunk<KV, NQB>(B, st, qf, c, kv_begin, kv_end, vis_end, edge_end, s_log2, ln);
          c += kChunk;
          if (c >= kv_end) break;
        }
      } else {
        while (true) {
          int cn = c + kChunk;
          bool more = cn < kv_end;
          if (more) issue(B, true);
          compute_chunk<KV, NQB>(A, st, qf, c, kv_begin, kv_end, vis_end, edge_end, s_log2, ln);
          c = cn;
          if (!more) break;
          cn = c + kChunk;
          more = cn < kv_end;
          if (more) issue(A, true);
          compute_chunk<KV, NQB>(B, st, qf, c, kv_begin, kv_end, vis_end, edge_end, s_log2, ln);
          c = cn;
          if (!more) break;
        }
      }
    }

    // express the partial against the true max: m = max score, l and o scaled to match; o also
    // takes the V scale of an 8-bit cache
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) {
      const float to_true = (st[cb].m_true == -INFINITY) ? 0.f : fast_exp2(st[cb].m_ref - st[cb].m_true);
      const float o_mul = to_true * o_scale;
#pragma unroll
      for (int n = 0; n < 8; ++n) st[cb].o[n] *= o_mul;
      float l = st[cb].l * to_true;
      l += xor_lane(l, 16);
      l += xor_lane(l, 32);
      const int row = ROWS > 1 ? 2 * cb + (ln.r >> 3) : (ln.r >> 3);
      if (row < q_len) {
        const size_t slot = ((size_t)s * (ROWS > 1 ? p.R : 1) + row) * p.Hq + h * 8 + (ln.r & 7);
        if (ln.grp == 0) {
          p.part_m[slot] = (st[cb].m_true == -INFINITY) ? -INFINITY : st[cb].m_true * kLn2;
          p.part_l[slot] = l;
        }
        float* dst = p.part_o + slot * kD + 4 * ln.grp;
#pragma unroll
        for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4*>(dst + 16 * n) = st[cb].o[n];
      }
    }
  }
  };

  if constexpr (!CLAIM) {
    // version 3 asks for list-major order: every workgroup of list w on XCD w mod 8 (b mod 8)
    if (version == LBSA_MAP_VERSION_PLACED)
      run_list(blockIdx.x % p.W, (blockIdx.x / p.W) * WAVES + wave);
    else
      run_list(blockIdx.x / G, (blockIdx.x % G) * WAVES + wave);
  } else {
    // workgroup b starts with item b; each further item takes one device-scope atomic on the
    // counter (issued by lane 0 as a vector memory atomic, broadcast), numbered after the grid's
    // first items, so no atomics at all are issued while the grid starts
    const int items = p.W * G;
    auto claim = [&]() __attribute__((always_inline)) {
      int v = 0;
      if (lane == 0) v = atomicAdd(p.claim, 1);
      return (int)gridDim.x + __builtin_amdgcn_readlane(v, 0);
    };
    for (int item = blockIdx.x; item < items; item = claim()) run_list(item / G, item % G);
    // every claim of this workgroup has returned; the last workgroup to get here resets the state
    if (lane == 0) {
      const int done = atomicAdd(p.claim + 1, 1);
      if (done == (int)gridDim.x - 1) {
        atomicExch(p.claim, 0);
        atomicExch(p.claim + 1, 0);
      }
    }
  }

  // loads of an empty last chunk may still be outstanding; drain them before the wave ends
  // (gfx9 s_waitcnt encoding: vmcnt 0, expcnt and lgkmcnt at their maximum)
  if constexpr (KV::kIssuePastEnd) __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));

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

template <class KV, int WAVES, int ROWS>
hipError_t launch_decode(const DecodeParams& p, int grid, hipStream_t stream) {
  if constexpr (WAVES == 1 && ROWS == 1) {
    if (p.claim) {
      hipLaunchKernelGGL((splitkv_decode_kernel<KV, 1, 1, true>), dim3(grid), dim3(64), 0, stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((splitkv_decode_kernel<KV, WAVES, ROWS>), dim3(grid), dim3(64 * WAVES), 0, stream, p);
  return hipGetLastError();
}

template <class KV, int ROWS>
hipError_t launch_waves(const DecodeParams& p, int waves, int grid, hipStream_t stream) {
  switch (waves) {
    case 1: return launch_decode<KV, 1, ROWS>(p, grid, stream);
    case 2: return launch_decode<KV, 2, ROWS>(p, grid, stream);
    case 4: return launch_decode<KV, 4, ROWS>(p, grid, stream);
    default: return launch_decode<KV, 8, ROWS>(p, grid, stream);
  }
}

template <class KV, int WAVES>
int decode_blocks_per_cu() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, splitkv_decode_kernel<KV, WAVES, 1>, 64 * WAVES, 0) !=
      hipSuccess)
    return 0;
  return nb;
}

// rows_per_unit = 1 with q_lens == null: plain decode; otherwise multi-token decode with up to
// rows_per_unit (<= 4) query rows per request.
template <class KV>
int splitkv_launch(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                   const float* v_scale, const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                   const int32_t* q_lens, const int32_t* q_start, const int32_t* seq_lens, const int32_t* map,
                   int32_t num_workers, int32_t num_segments, int32_t head_groups, int32_t B, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t rows_per_unit,
                   float softmax_scale, float* part_m, float* part_l, float* part_o, uint64_t* timing,
                   void* stream, int32_t* claim = nullptr, int32_t resident = 0) {
  if (num_workers < 1 || num_segments < 0 || B < 0 || head_groups < 1 || num_kv_heads < 1 ||
      num_pages < 1 || block_table_stride < 0 || page_size < 1 || rows_per_unit < 1)
    return LBSA_ERR_INVALID;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !map) return LBSA_ERR_INVALID;
  if ((q_lens == nullptr) != (q_start == nullptr)) return LBSA_ERR_INVALID;
  if (!q_lens && rows_per_unit != 1) return LBSA_ERR_INVALID;
  if (num_segments > 0 && (!part_m || !part_l || !part_o)) return LBSA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(part_o)) & 15)
    return LBSA_ERR_INVALID;
  if (head_dim != kD || num_q_heads != 8 * num_kv_heads || page_size % kMinPage != 0 || rows_per_unit > 4)
    return LBSA_ERR_UNSUPPORTED;
  if (num_kv_heads % head_groups) return LBSA_ERR_INVALID;
  const int waves = num_kv_heads / head_groups;
  if (waves != 1 && waves != 2 && waves != 4 && waves != 8) return LBSA_ERR_UNSUPPORTED;
  // one (page, KV head) block must stay addressable by a 32-bit buffer descriptor
  if ((int64_t)page_size * kD * KV::kElem > INT32_MAX) return LBSA_ERR_UNSUPPORTED;

  DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint8_t*>(k_cache);
  p.v = static_cast<const uint8_t*>(v_cache);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.map = map;
  p.part_m = part_m;
  p.part_l = part_l;
  p.part_o = part_o;
  p.q_lens = q_lens;
  p.q_start = q_start;
  p.timing = timing;
  p.claim = claim;
  p.G = head_groups;
  p.bt_stride = block_table_stride;
  p.num_pages = num_pages;
  p.W = num_workers;
  p.S = num_segments;
  p.B = B;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.page = page_size;
  p.R = rows_per_unit;
  p.scale_log2 = softmax_scale * kLog2e;

  if (claim && (waves != 1 || q_lens || resident < 1)) return LBSA_ERR_INVALID;
  const int64_t grid = claim ? (int64_t)resident : (int64_t)num_workers * head_groups;
  if (grid > INT32_MAX || (int64_t)num_workers * head_groups > INT32_MAX) return LBSA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (!q_lens)
    err = launch_waves<KV, 1>(p, waves, (int)grid, st);
  else if (rows_per_unit <= 2)
    err = launch_waves<KV, 2>(p, waves, (int)grid, st);
  else
    err = launch_waves<KV, 4>(p, waves, (int)grid, st);
  return err == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}

template <class KV>
int blocks_per_cu(int waves) {
  switch (waves) {
    case 1: return decode_blocks_per_cu<KV, 1>();
    case 2: return decode_blocks_per_cu<KV, 2>();
    case 4: return decode_blocks_per_cu<KV, 4>();
    default: return decode_blocks_per_cu<KV, 8>();
  }
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
  return splitkv_launch<KvBf16>(q, k_cache, v_cache, nullptr, nullptr, block_table, block_table_stride, num_pages,
                                nullptr, nullptr, seq_lens, map, num_workers, num_segments, head_groups, B,
                                num_q_heads, num_kv_heads, head_dim, page_size, 1, softmax_scale, part_m, part_l,
                                part_o, timing, stream);
}

extern "C" int attn_splitkv_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                                const float* v_scale, const int32_t* block_table, int32_t block_table_stride,
                                int32_t num_pages, const int32_t* seq_lens, const int32_t* map,
                                int32_t num_workers, int32_t num_segments, int32_t head_groups, int32_t B,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                float softmax_scale, float* part_m, float* part_l, float* part_o,
                                uint64_t* timing, void* stream) {
  if (!k_scale || !v_scale) return LBSA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3) return LBSA_ERR_INVALID;
  return splitkv_launch<KvFp8>(q, k_cache, v_cache, k_scale, v_scale, block_table, block_table_stride, num_pages,
                               nullptr, nullptr, seq_lens, map, num_workers, num_segments, head_groups, B,
                               num_q_heads, num_kv_heads, head_dim, page_size, 1, softmax_scale, part_m, part_l,
                               part_o, timing, stream);
}

extern "C" int attn_splitkv_mtp(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                const float* k_scale, const float* v_scale, const int32_t* block_table,
                                int32_t block_table_stride, int32_t num_pages, const int32_t* q_lens,
                                const int32_t* q_start, const int32_t* kv_lens, const int32_t* map,
                                int32_t num_workers, int32_t num_segments, int32_t head_groups, int32_t B,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                int32_t rows_per_unit, float softmax_scale, float* part_m, float* part_l,
                                float* part_o, void* stream) {
  if (!q_lens || !q_start) return LBSA_ERR_INVALID;
  if (kv_dtype == LBSA_KV_BF16) {
    if (k_scale || v_scale) return LBSA_ERR_INVALID;
    return splitkv_launch<KvBf16>(q, k_cache, v_cache, nullptr, nullptr, block_table, block_table_stride,
                                  num_pages, q_lens, q_start, kv_lens, map, num_workers, num_segments, head_groups,
                                  B, num_q_heads, num_kv_heads, head_dim, page_size, rows_per_unit, softmax_scale,
                                  part_m, part_l, part_o, nullptr, stream);
  }
  if (kv_dtype != LBSA_KV_FP8_E4M3) return LBSA_ERR_INVALID;
  if (!k_scale || !v_scale) return LBSA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3) return LBSA_ERR_INVALID;
  return splitkv_launch<KvFp8>(q, k_cache, v_cache, k_scale, v_scale, block_table, block_table_stride, num_pages,
                               q_lens, q_start, kv_lens, map, num_workers, num_segments, head_groups, B,
                               num_q_heads, num_kv_heads, head_dim, page_size, rows_per_unit, softmax_scale, part_m,
                               part_l, part_o, nullptr, stream);
}

extern "C" int attn_splitkv_claimed(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                    const float* k_scale, const float* v_scale, const int32_t* block_table,
                                    int32_t block_table_stride, int32_t num_pages, const int32_t* seq_lens,
                                    const int32_t* map, int32_t num_workers, int32_t num_segments,
                                    int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t page_size, float softmax_scale, int32_t resident_workgroups,
                                    int32_t* claim_state, float* part_m, float* part_l, float* part_o,
                                    uint64_t* timing, void* stream) {
  if (!claim_state || (reinterpret_cast<uintptr_t>(claim_state) & 3) || resident_workgroups < 1)
    return LBSA_ERR_INVALID;
  if (kv_dtype == LBSA_KV_BF16) {
    if (k_scale || v_scale) return LBSA_ERR_INVALID;
    return splitkv_launch<KvBf16>(q, k_cache, v_cache, nullptr, nullptr, block_table, block_table_stride,
                                  num_pages, nullptr, nullptr, seq_lens, map, num_workers, num_segments, num_kv_heads,
                                  B, num_q_heads, num_kv_heads, head_dim, page_size, 1, softmax_scale, part_m,
                                  part_l, part_o, timing, stream, claim_state, resident_workgroups);
  }
  if (kv_dtype != LBSA_KV_FP8_E4M3 || !k_scale || !v_scale) return LBSA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3) return LBSA_ERR_INVALID;
  return splitkv_launch<KvFp8>(q, k_cache, v_cache, k_scale, v_scale, block_table, block_table_stride, num_pages,
                               nullptr, nullptr, seq_lens, map, num_workers, num_segments, num_kv_heads, B,
                               num_q_heads, num_kv_heads, head_dim, page_size, 1, softmax_scale, part_m, part_l,
                               part_o, timing, stream, claim_state, resident_workgroups);
}

extern "C" int attn_query_workers(int device, int32_t head_groups, int32_t kv_dtype, int32_t* num_workers_out) {
  // per (device, cache type, head groups); atomics so that host threads may query at once (each
  // computes the same value)
  static std::atomic<int> cached[64][2][9];
  if (!num_workers_out || head_groups < 1 || head_groups > 8 || (8 % head_groups) || device < 0 ||
      device >= 64)
    return LBSA_ERR_INVALID;
  if (kv_dtype != LBSA_KV_BF16 && kv_dtype != LBSA_KV_FP8_E4M3) return LBSA_ERR_INVALID;
  const int known = cached[device][kv_dtype][head_groups].load(std::memory_order_relaxed);
  if (known > 0) {
    *num_workers_out = known;
    return LBSA_OK;
  }
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return LBSA_ERR_HIP;
  if (hipSetDevice(device) != hipSuccess) return LBSA_ERR_HIP;
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  const int waves = 8 / head_groups;
  int nb = 0;
  if (e == hipSuccess) nb = kv_dtype == LBSA_KV_BF16 ? blocks_per_cu<KvBf16>(waves) : blocks_per_cu<KvFp8>(waves);
  if (hipSetDevice(prev) != hipSuccess) return LBSA_ERR_HIP;
  if (e != hipSuccess || nb < 1 || cus < 1) return LBSA_ERR_HIP;
  const int w = cus * nb / head_groups;
  cached[device][kv_dtype][head_groups].store(w, std::memory_order_relaxed);
  *num_workers_out = w;
  return LBSA_OK;
}

// ---- allocation-free decode step ------------------------------------------------------------
//
// attn_decode_noalloc runs the split-KV kernel and the combine kernel of one decode step with the
// partials kept in `scratch`, a fixed device array of this library, so the call allocates nothing.
// Device code never names the array: host code takes its device address once per device with
// hipGetSymbolAddress and passes that address to the kernels like any caller-owned buffer.

namespace lbsa {

static __device__ __align__(256) unsigned char scratch[LBSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];   // device address of scratch, per device

// The device address of `scratch` on `device`, taken with that device current on first use.
static int scratch_address(int device, unsigned char** out) {
  if (device < 0 || device >= kMaxDevices) return LBSA_ERR_INVALID;
  void* known = g_scratch_addr[device].load(std::memory_order_acquire);
  if (!known) {
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return LBSA_ERR_HIP;
    if (prev != device && hipSetDevice(device) != hipSuccess) return LBSA_ERR_HIP;
    const hipError_t e = hipGetSymbolAddress(&known, HIP_SYMBOL(scratch));
    if (prev != device && hipSetDevice(prev) != hipSuccess) return LBSA_ERR_HIP;
    if (e != hipSuccess || !known) return LBSA_ERR_HIP;
    g_scratch_addr[device].store(known, std::memory_order_release);   // same value from any thread
  }
  *out = static_cast<unsigned char*>(known);
  return LBSA_OK;
}

}  // namespace lbsa

extern "C" int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                                   int32_t block_table_stride, int32_t num_pages, const int32_t* seq_lens,
                                   const int32_t* map, int32_t num_workers, int32_t num_segments,
                                   int32_t head_groups, int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t page_size, float softmax_scale, int32_t max_splits,
                                   void* out, int32_t out_dtype, void* stream) {
  if (num_segments < 0 || num_q_heads < 1 || head_dim < 1 || B < 0 || !out) return LBSA_ERR_INVALID;
  // partials: o [S, Hq, D] at the start of scratch (16-byte aligned rows), then m [S, Hq], l [S, Hq]
  const uint64_t items = (uint64_t)num_segments * (uint64_t)num_q_heads;
  const uint64_t need = items * ((uint64_t)head_dim + 2) * sizeof(float);
  if (need > LBSA_NOALLOC_SCRATCH_BYTES) return LBSA_ERR_CAPACITY;
  int device = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (st ? hipStreamGetDevice(st, &device) != hipSuccess : hipGetDevice(&device) != hipSuccess)
    return LBSA_ERR_HIP;
  unsigned char* base = nullptr;
  const int rc = scratch_address(device, &base);
  if (rc != LBSA_OK) return rc;
  float* part_o = reinterpret_cast<float*>(base);
  float* part_m = part_o + items * head_dim;
  float* part_l = part_m + items;
  int status;
  if (kv_dtype == LBSA_KV_BF16) {
    if (k_scale || v_scale) return LBSA_ERR_INVALID;
    status = splitkv_launch<KvBf16>(q, k_cache, v_cache, nullptr, nullptr, block_table, block_table_stride,
                                    num_pages, nullptr, nullptr, seq_lens, map, num_workers, num_segments,
                                    head_groups, B, num_q_heads, num_kv_heads, head_dim, page_size, 1,
                                    softmax_scale, part_m, part_l, part_o, nullptr, stream);
  } else if (kv_dtype == LBSA_KV_FP8_E4M3) {
    if (!k_scale || !v_scale) return LBSA_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3) return LBSA_ERR_INVALID;
    status = splitkv_launch<KvFp8>(q, k_cache, v_cache, k_scale, v_scale, block_table, block_table_stride,
                                   num_pages, nullptr, nullptr, seq_lens, map, num_workers, num_segments,
                                   head_groups, B, num_q_heads, num_kv_heads, head_dim, page_size, 1,
                                   softmax_scale, part_m, part_l, part_o, nullptr, stream);
  } else {
    return LBSA_ERR_INVALID;
  }
  if (status != LBSA_OK) return status;
  // decode maps have one unit per request
  return attn_combine(part_m, part_l, part_o, map, B, 1, nullptr, nullptr, num_q_heads, head_dim, out, out_dtype,
                      max_splits, stream);
}
