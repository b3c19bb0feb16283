// Split-KV chunked prefill over a cached prefix, driven by the same greedy work map.
//
// The pages' load-balanced scheduler ([P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案;
// [P4] "腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级" §二.1) applied to prefill units: a unit
// is a 256-row (or 128-row) block of one request's query chunk, cut into 512-token KV tiles that the
// planner packs onto workers exactly as in decode.  Prefix-cache reuse ([P3] §6) means each chunk
// attends to a long cached prefix plus itself under a causal mask: row j of a q_len-row chunk sits at
// position kv_len - q_len + j and sees keys [0, that position].
//
// gfx950 design.  Workgroup = (worker w, KV head g, HPW query heads of the group), 8 waves, each
// owning 32 query rows of one head: 256-row units run one head per workgroup (wave v has rows
// 32v .. 32v+31), 128-row units two heads (waves 0-3 the first, 4-7 the second).  Each 64-key chunk
// of K and V (blocked cache layout) goes from HBM straight into LDS with buffer->LDS loads (no
// registers), in XOR-swizzled layouts that the MFMA fragment reads take without bank conflicts, and
// is read by every wave: 256 (query row, head) columns per K/V load at either unit height, so the
// staging and the fp16 conversion of V are shared by all of them; the workgroups covering the eight
// query heads of a KV head run on one XCD so K/V come from one L2.  Two 32 KiB LDS stages (the next
// chunk streams in while the current one is computed) and a register budget of 256 give two waves
// per SIMD (one workgroup per CU), so one wave's softmax VALU work can overlap another wave's MFMAs.
// Per wave, with the query rows as the MFMA columns:
//   S^T (keys x rows) = K . Q^T       v_mfma_f32_16x16x32_bf16, Q^T fragments held in VGPRs
//   O^T (dims x rows) += V^T . P^T    fp16 operands (V converted in LDS), or bf16 with P as
//                                      hi + lo parts (see "P.V precision" below)
// so every lane holds whole columns: the softmax max/sum of a row needs only in-lane reductions and
// two lane exchanges, exactly as in the decode kernel.  Key tiles are interleaved in 4-key groups so
// that a lane's 8 scores per 32 keys are the 8 consecutive keys it supplies to the PV product.

#include "common.h"
#include "lbsa.h"

namespace lbsa {

struct PrefillParams {
  const uint16_t* q;            // [rows, Hq, 128]
  const uint16_t* k;            // [pages, Hkv] blocks: [4][page][32] (dim tile, key, dim)
  const uint16_t* v;            // [pages, Hkv] blocks: [page / 32][128][32] (key tile, dim, key)
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
constexpr int kRow = 64;          // bytes per row of the blocked cache layout
constexpr int kPChunk = 64;       // keys per staged chunk
constexpr int kMaxQTile = 256;    // query rows per unit: 32 per wave, 4 or 8 waves per query head
constexpr int kColBlocks = 2;     // 16-row column blocks per wave (32 rows)
constexpr int kKRow = kPD * 2;             // LDS bytes per key row of K (16 granules, XOR-swizzled)
constexpr int kVRow = kPChunk * 2;         // LDS bytes per dim row of V^T (8 granules, XOR-swizzled)
constexpr int kKBytes = kPChunk * kKRow;   // 16 KiB
constexpr int kVBytes = kPD * kVRow;       // 16 KiB
constexpr int kStage = kKBytes + kVBytes;  // one pipeline stage: a 64-key chunk of K and V^T
constexpr float kPRescaleSlack = 8.0f;   // log2 units

// Tuning knobs (compile-time):
//
// P.V precision (runtime, template parameter PV):
//   kPvF16   each chunk's V^T is converted to fp16 once, in LDS, by the workgroup (each thread its
//            own copied granules, before the chunk's barrier) and P is rounded to fp16 (11
//            significant bits); the products run on v_mfma_f32_16x16x32_f16.  The conversion
//            rounds toward zero: exact for v = 0 and 2^-17 <= |v| <= 65504 (every bf16 value there
//            has at most fp16's bits); smaller magnitudes lose low bits in fp16's subnormals and
//            vanish below 2^-24, larger ones saturate at 65504.
//   kPvExact bf16 V with P split into bf16 hi + lo parts (two MFMAs, ~16 significant bits): exact
//            for every bf16 V.
//   kPvGuard (default) the fp16 path on V * 2^6 and P * 2^-6 (the products are unchanged), except
//            that the conversion also checks every V value of the chunk: a chunk holding any value
//            outside 2^-23 <= |v| <= 1020 (where fp16 carries bf16 * 2^6 exactly; exact zeros are
//            sent along with them) is stamped, and its P.V takes the exact path with V^T read from
//            the cache.  V is then carried exactly for every bf16 input, at the fp16 path's speed
//            whenever the values fit.  The shift centres fp16's window on activation magnitudes:
//            unshifted, any chunk holding a |v| below 2^-17 is stamped, ~5% of the chunks of
//            N(0, 1) V and nearly all of N(0, 0.02^2) V; shifted, ~0.1% and ~4%.
//   LBSA_PREFILL_WPE     waves per SIMD the register budget is fitted to (1 or 2)

#ifndef LBSA_PREFILL_WPE
#define LBSA_PREFILL_WPE 2
#endif

constexpr int kGuardShift = 6;   // guarded path: V carried as V * 2^6 in fp16, P as P * 2^-6

constexpr int kPvExact = 0;
constexpr int kPvGuard = 1;
constexpr int kPvF16 = 2;


typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));


// two bf16 values (one dword) -> two fp16 values, round toward zero: exact for 0 and
// 2^-17 <= |v| <= 65504; below that the fp16 subnormal spacing (2^-24) truncates, above it the value
// saturates at +-65504 instead of overflowing
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(x), bf16_hi(x)));
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Maximum of two scores.  Scores are finite or -inf (masked keys are selected to -inf, never
// computed from padding), so the NaN-propagating maximum gives the same result as fmaxf; unlike
// fmaxf it needs no quieting of its inputs and maps to gfx950's v_maximum3_f32.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// maximum of v over lanes l, l ^ 16, l ^ 32 and l ^ 48 (one value from each 16-lane row): gfx950's
// row-swap permutes exchange the two halves of the wave, then rows 0/1 and 2/3, as VALU operations
__device__ __forceinline__ float max_over_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float m = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ u32x4 lds_ld16(const uint8_t* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// K rows are 256 B (16 granules).  The 16 lanes of one ds_read_b128 read the same granule of keys
// {0-3, 8-11, 16-19, 24-27} (+4): granule G of key k sits at slot G ^ swz(k), which gives those 16
// keys 16 different bank groups.
__device__ __forceinline__ int k_swz(int key) { return (key & 3) | (((key >> 3) & 3) << 2); }
__device__ __forceinline__ int k_slot(int key, int granule) { return key * kKRow + 16 * (granule ^ k_swz(key)); }

// V^T rows are 128 B (8 granules).  The 16 lanes of one read take dims 16n + 0..15 at one key
// granule: granule G of dim d sits at slot G ^ ((d >> 1) & 7), so the 16 reads hit 16 bank groups.
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }
__device__ __forceinline__ int v_slot(int d, int granule) { return kKBytes + d * kVRow + 16 * (granule ^ v_swz(d)); }

#define LBSA_LDS(ptr) ((__attribute__((address_space(3))) void*)(ptr))

// Buffer resource of `bytes` bytes at p (stride 0, raw buffer): base, num_records, flags.
__device__ __forceinline__ u32x4 raw_rsrc(const void* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, (uint32_t)bytes, 0x00020000u};
}

// Copy of 16 bytes per lane from a buffer straight into LDS (the 64 lanes fill 1 KiB at LDS address
// lds), written as inline assembly on purpose: with copies still in flight across the loop, the
// compiler's wait-count pass no longer tells the LDS stages apart and would make every LDS read wait
// for all outstanding copies.  The kernel waits for its own copies (vmcnt) and publishes them with
// a barrier before any wave reads them; the memory clobber keeps LDS accesses in program order
// around the copy.  The LDS address goes in as an operand bound to M0, so the compiler sets M0
// itself and knows its value; the s_nop gives the M0 write the wait state the copy needs.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, const uint8_t* lds, int voff, int soff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LBSA_LDS(lds)));
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0)
               : "memory");
}

// Read-only kernel inputs read at wave-uniform addresses (block table): the constant address
// space makes them scalar loads, counted apart from the vector-memory queue the LDS DMA uses.
typedef const __attribute__((address_space(4))) int32_t const_i32;

// s_waitcnt with vmcnt <= vm and lgkmcnt <= lgkm (gfx9 encoding; expcnt left at its maximum)
#define LBSA_WAIT_VM_LGKM(vm, lgkm) \
  __builtin_amdgcn_s_waitcnt(((vm) & 0xF) | (((vm) >> 4) << 14) | (0x7 << 4) | (((lgkm) & 0xF) << 8))

// Unit height and DMA share of a workgroup of WAVES waves (a struct, not function-local constants:
// the host pass of the kernel template needs them as constant expressions).
template <int WAVES, int HPW>
struct PrefillShape {
  static constexpr int kWavesPerHead = WAVES / HPW;
  static constexpr int kQTile = 32 * kWavesPerHead;   // query rows per unit
  static constexpr int kTpw = 16 / WAVES;             // 1 KiB DMA slots per wave in each half of a stage
  static constexpr int kGroups = 8 / HPW;             // workgroups per (worker, KV head)
};

template <int PV, int WAVES, int HPW = 1>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(LBSA_PREFILL_WPE, LBSA_PREFILL_WPE)))
void splitkv_prefill_kernel(PrefillParams p) {
  using Shape = PrefillShape<WAVES, HPW>;
  // exponent shift of the fp16 operands: V * 2^kShift and P * 2^-kShift (guarded path only)
  constexpr int kShift = PV == kPvGuard ? kGuardShift : 0;
  // the pipeline stages, separate objects so the compiler can tell their DMA writes apart
  __shared__ __attribute__((aligned(16))) uint8_t stage0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;
  const int grp = lane >> 4;

  // block -> (worker, KV head, query heads of the group); the 8 / HPW workgroups of one
  // (worker, KV head) land on the same XCD (dispatch is round-robin over 8 XCDs) and are
  // dispatched together, so the K/V they share comes from one L2
  const int f = blockIdx.x;
  const int xcd = f & 7;
  const int kq = f >> 3;
  const int hq = kq % Shape::kGroups;
  const int wg_index = (kq / Shape::kGroups) * 8 + xcd;      // (w * Hkv + g)
  const int w = wg_index / p.Hkv;
  const int g = wg_index - w * p.Hkv;
  if (w >= p.W) return;
  // query head of this wave (a workgroup runs HPW query heads of the group, WAVES / HPW waves each)
  const int h = g * 8 + hq * HPW + wave / Shape::kWavesPerHead;
  const int rbase = 32 * (wave % Shape::kWavesPerHead);   // first row (inside the unit) of this wave

  const_i32* map = (const_i32*)p.map;
  if (map[0] != LBSA_MAP_VERSION) return;   // a device-built map that reported an error
  if (map[6] != Shape::kQTile) return;              // a map planned for another unit height
  if (map[2] != p.W) return;                        // a map planned for another worker count
  const int U = map[7];
  const_i32* worker_ptr = map + 8;
  const_i32* segs = map + 8 + (p.W + 1) + (U + 1) + 2 * U;
  const_i32* q_lens = (const_i32*)p.q_lens;
  const_i32* q_start = (const_i32*)p.q_start;
  const_i32* kv_lens = (const_i32*)p.kv_lens;
  const int s_begin = worker_ptr[w];
  const int s_end = min(worker_ptr[w + 1], p.S);
  const int block_bytes = p.page * kPD * 2;
  const float c = p.scale_log2;                 // raw score -> log2 units
  const float slack_raw = kPRescaleSlack / c;

  // DMA layout: wave v fills LDS granules 64*(kTpw*v + t) + lane, t < kTpw (2 with eight waves), of
  // the K half and of the V^T half of a stage; the lane fetches whichever global granule belongs in
  // that swizzled slot
  // LDS fragment addresses.  K: key 32kb + 4j + key0 at granule 4ks + grp; the swizzle of those keys
  // is swz(key0) for every (kb, j), so each read is k_base[ks] + (32kb + 4j) * 256.  V^T: dim
  // 16n + r at granule 4kb + grp; the swizzle depends on r only, so each read is v_base[kb] + 2048n.
  const int key0 = 8 * (r >> 2) + (r & 3);
  int k_base[4], v_base[2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) k_base[ks] = k_slot(key0, 4 * ks + grp);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) v_base[kb] = v_slot(r, 4 * kb + grp);

  // byte offsets inside a (page, KV head) block of the blocked cache layout (rows of 64 bytes: K
  // [4 dim tiles][page keys][32 dims], V [page / 32 key tiles][128 dims][32 keys]); the chunk's
  // offset in the page goes in the scalar offset, so these registers stay unchanged while earlier
  // loads that read them are in flight.  LDS slot `slot` of the stage takes 16-byte piece kp of
  // key row `key` (dims 8kp .. +7) and piece vp of dim row d (chunk keys 8vp .. +7).
  int k_src[4], v_src[4];   // the first Shape::kTpw are used (a fixed size keeps the lambdas host-compilable)
#pragma unroll
  for (int t = 0; t < Shape::kTpw; ++t) {
    const int slot = 64 * (Shape::kTpw * wave + t) + lane;
    const int key = slot >> 4;
    const int kp = (slot & 15) ^ k_swz(key);
    k_src[t] = ((kp >> 2) * p.page + key) * kRow + 16 * (kp & 3);
    const int d = slot >> 3;
    const int vp = (slot & 7) ^ v_swz(d);
    v_src[t] = ((vp >> 2) * kPD + d) * kRow + 16 * (vp & 3);
  }

  // guarded fp16 P.V: stamp[stage] = running chunk number of the chunk in that stage whose V is not
  // held exactly by fp16 (set while converting it), so that the chunk's P.V takes the exact path
  __shared__ int stamp_mem[2];
  volatile int* stamp = stamp_mem;
  int gbase = 0;   // chunks staged by this workgroup in earlier segments
  if constexpr (PV == kPvGuard) {
    if (tid == 0) stamp[0] = stamp[1] = -1;
    __syncthreads();
  }

  for (int s = s_begin; s < s_end; ++s) {
    const int b = segs[4 * s];
    const int qt = segs[4 * s + 1];
    const int kv_begin = max(segs[4 * s + 2], 0);
    int kv_end = segs[4 * s + 3];
    if (b < 0 || b >= p.B) continue;
    const int q_len = q_lens[b];
    const int kv_len = kv_lens[b];
    const int prefix = kv_len - q_len;
    kv_end = min(kv_end, kv_len);
    kv_end = min(kv_end, p.bt_stride * p.page);
    const int unit_row0 = qt * Shape::kQTile;                 // first row of the unit inside the chunk
    const int wave_row0 = unit_row0 + rbase;           // first row of this wave
    // last key any row of this wave may see (-1: the wave has no row inside the chunk); the wave's
    // rows are wave_row0 .. wave_row0 + 16 * kColBlocks - 1
    const int wave_last_key = wave_row0 >= q_len ? -1
                              : (p.causal ? prefix + min(wave_row0 + 16 * kColBlocks - 1, q_len - 1) : kv_len - 1);

    // Q^T fragments: column r of block cb = row wave_row0 + 16cb + r, k = dims 32ks + 8grp .. +7
    u32x4 qf[kColBlocks][4];
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      const int row = wave_row0 + 16 * cb + r;
      const bool ok = row < q_len;
      const uint16_t* qp = p.q + ((size_t)(q_start[b] + (ok ? row : 0)) * p.Hq + h) * kPD + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[cb][ks] = ok ? ld16(qp + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
    }
    // Q has landed before any K/V copy is issued: the copies are invisible to the compiler, whose own
    // wait for Q would otherwise wait for every copy in flight too
    LBSA_WAIT_VM_LGKM(0, 15);

    // reference maximum (raw score units), true maximum, row sum, and -m_ref in log2 units (0 while
    // m_ref is -inf) per column block
    float m_ref[kColBlocks], m_true[kColBlocks], lsum[kColBlocks], neg_mc[kColBlocks];
    f32x4 o[kColBlocks][8];
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      m_ref[cb] = -INFINITY;
      m_true[cb] = -INFINITY;
      lsum[cb] = 0.f;
      neg_mc[cb] = 0.f;
#pragma unroll
      for (int n = 0; n < 8; ++n) o[cb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const_i32* bt_row = (const_i32*)(p.block_table + (size_t)b * p.bt_stride);
    const int c_first = kv_begin & ~(kPChunk - 1);
    const int n_chunks = kv_end > c_first ? (kv_end - c_first + kPChunk - 1) / kPChunk : 0;

    // chunk i -> stage: each wave issues 2 * kTpw buffer->LDS loads of 1 KiB (kTpw of K, kTpw of V^T)
    auto dma = [&](int i, uint8_t* st) __attribute__((always_inline)) {
      const int c0 = c_first + kPChunk * i;
      const int pg = c0 / p.page;
      const int off = c0 - pg * p.page;
      int pid = bt_row[pg];
      pid = min(max(pid, 0), p.num_pages - 1);
      const size_t blk = ((size_t)pid * p.Hkv + g) * (size_t)p.page * kPD;
      const u32x4 kr = raw_rsrc(p.k + blk, block_bytes);
      const u32x4 vr = raw_rsrc(p.v + blk, block_bytes);
#pragma unroll
      for (int t = 0; t < Shape::kTpw; ++t) lds_dma16(kr, st + 1024 * (Shape::kTpw * wave + t), k_src[t], off * kRow);
#pragma unroll
      for (int t = 0; t < Shape::kTpw; ++t)
        lds_dma16(vr, st + kKBytes + 1024 * (Shape::kTpw * wave + t), v_src[t], (off / 32) * kPD * kRow);
    };

    // a chunk needs masking if it holds keys outside [kv_begin, kv_end) or (causal) keys after the
    // position of some row of this wave
    auto chunk_edge = [&](int c0) __attribute__((always_inline)) {
      return (c0 < kv_begin) || (c0 + kPChunk > kv_end) || (p.causal && c0 + kPChunk - 1 > prefix + wave_row0);
    };
    // S^T of one 32-key block of the chunk in stage st: scb[cb][4j+i] = raw q.k of key
    // c0 + 32kb + 8grp + 4j + i and column (row) r of block cb; masked keys get -inf
    auto scores = [&](int c0, bool edge, const uint8_t* st, int kb, float (&scb)[kColBlocks][8]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 kf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[ks] = lds_ld16(st, k_base[ks] + (32 * kb + 4 * j) * kKRow);
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(kf[ks], qf[cb][ks], acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) scb[cb][4 * j + e] = acc[e];   // raw q.k; scaled inside exp2
        }
      }
      if (edge) {
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb) {
          const int row = wave_row0 + 16 * cb + r;
          const int last = p.causal ? prefix + row : kv_len - 1;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = c0 + 32 * kb + 8 * grp + e;
            scb[cb][e] = (t < kv_begin || t >= kv_end || t > last) ? -INFINITY : scb[cb][e];
          }
        }
      }
    };
    // maximum of a chunk's 64 scores per row (column): mxs, the running true maximum, and whether
    // this lane's rows pass their reference maximum by more than the slack
    auto chunk_max = [&](const float (&sc)[2][kColBlocks][8], float (&mxs)[kColBlocks]) __attribute__((always_inline)) {
      bool any_rescale = false;
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) {
        float mx = sc[0][cb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 8; ++e) mx = vmax(mx, sc[kb][cb][e]);
        mx = max_over_rows(mx);
        m_true[cb] = vmax(m_true[cb], mx);
        mxs[cb] = mx;
        any_rescale |= mx > m_ref[cb] + slack_raw;
      }
      return any_rescale;
    };
    // move the reference maximum of the rows whose chunk maximum passed it (0 from -inf), rescaling
    // their accumulators and row sums; the others keep theirs, which may still be -inf for a row
    // with no visible key yet (-inf - -inf would be NaN)
    auto rescale_to = [&](const float (&mxs)[kColBlocks]) __attribute__((always_inline)) {
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) {
        const bool move = mxs[cb] > m_ref[cb] + slack_raw;
        const float m_new = move ? mxs[cb] : m_ref[cb];
        const float alpha = move ? fast_exp2((m_ref[cb] - m_new) * c) : 1.f;
        m_ref[cb] = m_new;
        neg_mc[cb] = move ? -m_new * c - (float)kShift : neg_mc[cb];
        lsum[cb] *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) o[cb][n] *= alpha;
      }
    };
    // probabilities of a chunk against the reference maximum, their row sums, and P packed as the B
    // operand of the P.V products (fp16; or bf16 hi + lo parts)
    // (fp16 path: the row sums add the fp16-rounded probabilities, the very values the P.V products
    // take, two per v_dot2_f32_f16 against (1, 1) with fp32 accumulation)
    auto exp_pack = [&](const float (&sc)[2][kColBlocks][8], u32x4 (&pf)[2][kColBlocks][2], bool f16) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb) {
          float ps[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) ps[e] = fast_exp2(fmaf(sc[kb][cb][e], c, neg_mc[cb]));
          if (f16) {
            const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // (the sum reads the packed pair itself: reading the element back through pf was
              // compiled to the first element's register for every e)
              const f16x2 ph = {(_Float16)ps[2 * e], (_Float16)ps[2 * e + 1]};
              pf[kb][cb][0][e] = __builtin_bit_cast(uint32_t, ph);
              lsum[cb] = __builtin_amdgcn_fdot2(ph, ones, lsum[cb], false);
            }
          } else {
            // P split into bf16 hi + lo parts: two MFMAs keep ~16 significant bits of each probability
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lsum[cb] += ps[2 * e] + ps[2 * e + 1];
              const uint32_t hv = pack_bf16(ps[2 * e], ps[2 * e + 1]);
              pf[kb][cb][0][e] = hv;
              pf[kb][cb][1][e] = pack_bf16(ps[2 * e] - bf16_lo(hv), ps[2 * e + 1] - bf16_hi(hv));
            }
          }
        }
      }
    };
    // one online-softmax update over the 64 scores of a chunk
    auto softmax_chunk = [&](const float (&sc)[2][kColBlocks][8], u32x4 (&pf)[2][kColBlocks][2], bool f16) __attribute__((always_inline)) {
      float mxs[kColBlocks];
      if (__builtin_amdgcn_ballot_w64(chunk_max(sc, mxs))) rescale_to(mxs);
      exp_pack(sc, pf, f16);
    };
    // O^T += V^T . P^T for the chunk in stage st
    // (vedge: the chunk holds keys outside [kv_begin, kv_end), whose V must be masked)
    auto v_edge = [&](int c0) __attribute__((always_inline)) { return (c0 < kv_begin) || (c0 + kPChunk > kv_end); };
    // O^T += V^T . P^T for 32-key block kb of the chunk in stage st
    auto pv_block = [&](int c0, bool vedge, const uint8_t* st, int kb, const u32x4 (&pb)[kColBlocks][2], bool f16) __attribute__((always_inline)) {
      const int kbase = c0 + 32 * kb;
      // V^T fragments of this 32-key block: dim 16n + r, keys kbase + 8grp .. +7
      u32x4 vf[8];
      if (PV == kPvGuard && !f16) {
        // the exact path of a guarded chunk: bf16 V^T straight from the cache (rare; the staged copy
        // holds the fp16 conversion): row (32-key tile, dim) of the chunk's (page, KV head) block
        const int pg = c0 / p.page;
        int pid = bt_row[pg];
        pid = min(max(pid, 0), p.num_pages - 1);
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(p.v) + ((size_t)pid * p.Hkv + g) * (size_t)block_bytes;
        const int tile = (c0 - pg * p.page + 32 * kb) / 32;
#pragma unroll
        for (int n = 0; n < 8; ++n) vf[n] = ld16(blk + (size_t)(tile * kPD + 16 * n + r) * kRow + 16 * grp);
      } else {
#pragma unroll
        for (int n = 0; n < 8; ++n) vf[n] = lds_ld16(st, v_base[kb] + 16 * n * kVRow);
      }
      if (vedge) {
        // keys outside [kv_begin, kv_end) may hold any bits; p = 0 does not cancel a NaN
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = kbase + 8 * grp + 2 * e;
          const uint32_t keep = ((t >= kv_begin && t < kv_end) ? 0x0000ffffu : 0u) |
                                ((t + 1 >= kv_begin && t + 1 < kv_end) ? 0xffff0000u : 0u);
#pragma unroll
          for (int n = 0; n < 8; ++n) vf[n][e] &= keep;
        }
      }
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) {
        if (f16) {
#pragma unroll
          for (int n = 0; n < 8; ++n) o[cb][n] = mfma16x16x32_f16(vf[n], pb[cb][0], o[cb][n]);
        } else {
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            o[cb][n] = mfma16x16x32(vf[n], pb[cb][0], o[cb][n]);
            o[cb][n] = mfma16x16x32(vf[n], pb[cb][1], o[cb][n]);
          }
        }
      }
    };
    // O^T += V^T . P^T for the chunk in stage st
    auto pv_chunk = [&](int c0, bool vedge, const uint8_t* st, const u32x4 (&pf)[2][kColBlocks][2], bool f16) __attribute__((always_inline)) {
      pv_block(c0, vedge, st, 0, pf[0], f16);
      pv_block(c0, vedge, st, 1, pf[1], f16);
    };
    // the whole chunk i in one wave: S^T, softmax, P.V
    auto compute = [&](int i, const uint8_t* st) __attribute__((always_inline)) {
      const int c0 = c_first + kPChunk * i;
      if (c0 > wave_last_key) return;   // chunk entirely past this wave's rows (causal) or no rows
      const bool edge = chunk_edge(c0);
      float sc[2][kColBlocks][8];
      // a wave issuing matrix products takes the SIMD's issue priority, so the other wave's softmax
      // fills the matrix core's shadow instead of contending with the products (~1% on every
      // configuration; the arithmetic is unchanged)
      __builtin_amdgcn_s_setprio(1);
      scores(c0, edge, st, 0, sc[0]);
      scores(c0, edge, st, 1, sc[1]);
      __builtin_amdgcn_s_setprio(0);
      // P.V in fp16 on the fp16 path, and on the guarded path unless the chunk's V was stamped
      const bool f16 = PV == kPvF16 || (PV == kPvGuard && stamp[st == stage0 ? 0 : 1] != gbase + i);
      if (PV != kPvGuard || f16) {
        u32x4 pf[2][kColBlocks][2];
        softmax_chunk(sc, pf, PV != kPvExact);
        __builtin_amdgcn_s_setprio(1);
        pv_chunk(c0, v_edge(c0), st, pf, PV != kPvExact);
        __builtin_amdgcn_s_setprio(0);
      } else {
        // exact P.V of a stamped chunk, one 32-key block at a time (hi + lo P of one block live)
        float mxs[kColBlocks];
        if (__builtin_amdgcn_ballot_w64(chunk_max(sc, mxs))) rescale_to(mxs);
        const bool vedge = v_edge(c0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          u32x4 pb[kColBlocks][2];
#pragma unroll
          for (int cb = 0; cb < kColBlocks; ++cb) {
            float ps[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ps[e] = fast_exp2(fmaf(sc[kb][cb][e], c, neg_mc[cb]));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // the row sums stay in the shifted units; the bf16 V products take P itself
              lsum[cb] += ps[2 * e] + ps[2 * e + 1];
              const float p0 = ps[2 * e] * (float)(1 << kShift), p1 = ps[2 * e + 1] * (float)(1 << kShift);
              const uint32_t hv = pack_bf16(p0, p1);
              pb[cb][0][e] = hv;
              pb[cb][1][e] = pack_bf16(p0 - bf16_lo(hv), p1 - bf16_hi(hv));
            }
          }
          pv_block(c0, vedge, st, kb, pb, false);
        }
      }
    };


    // V^T of the chunk in stage st: keys outside [kv_begin, kv_end) stay as loaded (the P.V
    // fragments mask them); on the fp16 path the values are converted to fp16 in place.  Each
    // thread converts the granules its own buffer->LDS loads wrote, so only its own loads need to
    // have landed.
    auto to_f16 = [&](uint8_t* st, int chunk) __attribute__((always_inline)) {
      // guarded path: the largest (|v| - 2^-23) as packed 16-bit bf16 patterns, wrapping below 2^-23
      u16x2 mx = {0, 0};
#pragma unroll
      for (int t = 0; t < Shape::kTpw; ++t) {
        u32x4* gp = reinterpret_cast<u32x4*>(st + kKBytes + 1024 * (Shape::kTpw * wave + t) + 16 * lane);
        u32x4 x = *gp;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (PV == kPvGuard) {
            const u16x2 a = __builtin_bit_cast(u16x2, x[e] & 0x7fff7fffu);
            constexpr unsigned short lo = 0x3700 - (kShift << 7);
            mx = __builtin_elementwise_max(mx, a - (u16x2){lo, lo});
          }
          // V * 2^kShift: the shift added to both exponent fields (a value outside the window,
          // whose field could carry over, is in a stamped chunk whose fp16 copy is not used)
          constexpr uint32_t up = (uint32_t)(kShift << 7) * 0x00010001u;
          x[e] = bf16x2_to_f16x2(x[e] + up);
        }
        *gp = x;
      }
      if constexpr (PV == kPvGuard) {
        // fp16 holds every bf16 value with 2^-17 <= |v| <= 65280 (bf16 0x3700 .. 0x477f) exactly, so
        // V * 2^6 for 2^-23 <= |v| <= 1020 (0x3400 .. 0x447f): |v| - 0x3400 lands in 0 .. 0x107f
        // for those and above it for any other value, 0 included (one comparison per value; a
        // chunk holding an exact 0 takes the exact path too)
        const bool bad = mx[0] > 0x107f || mx[1] > 0x107f;
        if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) stamp[st == stage0 ? 0 : 1] = gbase + chunk;
      }
    };
    // one pipeline step: start chunk i+1's DMA into the other stage (last read by chunk i-1,
    // finished by every wave before the previous barrier), compute chunk i, wait for the DMA,
    // convert chunk i+1's V (fp16 path), barrier: one barrier per chunk makes chunk i+1 ready for
    // every wave and releases chunk i's stage
    auto step = [&](int i, uint8_t* cur, uint8_t* ahead) __attribute__((always_inline)) {
      const bool more = i + 1 < n_chunks;
      if (more) dma(i + 1, ahead);
      compute(i, cur);
      if constexpr (PV != kPvExact) {
        if (more) {
          LBSA_WAIT_VM_LGKM(0, 15);
          to_f16(ahead, i + 1);
        }
      }
      LBSA_WAIT_VM_LGKM(0, 0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");   // the stamps and staged chunks read after the barrier stay after it
    };

    if (n_chunks > 0) {
      dma(0, stage0);
      if constexpr (PV != kPvExact) {
        LBSA_WAIT_VM_LGKM(0, 15);
        to_f16(stage0, 0);
      }
      LBSA_WAIT_VM_LGKM(0, 0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      for (int i = 0; i < n_chunks; i += 2) {
        step(i, stage0, stage1);
        if (i + 1 >= n_chunks) break;
        step(i + 1, stage1, stage0);
      }
      gbase += n_chunks;
    }

    // write the partials of this wave's rows (rows past the chunk's end are not stored)
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      const float to_true = (m_true[cb] == -INFINITY) ? 0.f : fast_exp2((m_ref[cb] - m_true[cb]) * c);
      float l = lsum[cb] * (to_true * (float)(1 << kShift));   // row sums back from the shifted units
      l += xor_lane(l, 16);
      l += xor_lane(l, 32);
      const int row_in_unit = rbase + 16 * cb + r;
      if (unit_row0 + row_in_unit < q_len) {
        const size_t slot = ((size_t)s * Shape::kQTile + row_in_unit) * p.Hq + h;
        if (grp == 0) {
          p.part_m[slot] = (m_true[cb] == -INFINITY) ? -INFINITY : m_true[cb] * c * kLn2;
          p.part_l[slot] = l;
        }
        float* dst = p.part_o + slot * kPD + 4 * grp;
#pragma unroll
        for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4*>(dst + 16 * n) = o[cb][n] * to_true;
      }
    }
  }
}

template <int PV, int WAVES, int HPW = 1>
void launch_prefill(unsigned grid, hipStream_t stream, const PrefillParams& p) {
  hipLaunchKernelGGL((splitkv_prefill_kernel<PV, WAVES, HPW>), dim3(grid), dim3(64 * WAVES), 0, stream, p);
}

}  // namespace lbsa

using namespace lbsa;

extern "C" int attn_splitkv_prefill(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                                    const int32_t* q_lens, const int32_t* q_start, const int32_t* kv_lens,
                                    const int32_t* map, int32_t num_workers, int32_t num_segments, int32_t B,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                    int32_t q_tile, int32_t causal, float softmax_scale, float* part_m,
                                    float* part_l, float* part_o, int32_t flags, void* stream) {
  if (num_workers < 1 || num_segments < 0 || B < 0 || num_kv_heads < 1 || num_pages < 1 ||
      block_table_stride < 0 || page_size < 1)
    return LBSA_ERR_INVALID;
  if (!q || !k_cache || !v_cache || !block_table || !q_lens || !q_start || !kv_lens || !map)
    return LBSA_ERR_INVALID;
  if (num_segments > 0 && (!part_m || !part_l || !part_o)) return LBSA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(part_o)) & 15)
    return LBSA_ERR_INVALID;
  if (head_dim != kPD || num_q_heads != 8 * num_kv_heads || page_size % kPChunk != 0 ||
      (q_tile != 128 && q_tile != kMaxQTile))
    return LBSA_ERR_UNSUPPORTED;
  if (flags & ~(LBSA_PREFILL_EXACT_PV | LBSA_PREFILL_F16_PV)) return LBSA_ERR_INVALID;
  if ((flags & LBSA_PREFILL_EXACT_PV) && (flags & LBSA_PREFILL_F16_PV)) return LBSA_ERR_INVALID;
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
  const int64_t grid128 = ((pairs + 7) / 8) * 8 * 4;   // 128-row units: two query heads per workgroup
  const int64_t grid = ((pairs + 7) / 8) * 8 * 8;
  if (grid > INT32_MAX) return LBSA_ERR_INVALID;
  const int mode = (flags & LBSA_PREFILL_EXACT_PV) ? kPvExact : (flags & LBSA_PREFILL_F16_PV) ? kPvF16 : kPvGuard;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned g = (unsigned)grid;
  if (q_tile == 128) {
    const unsigned g2 = (unsigned)grid128;
    if (mode == kPvExact) launch_prefill<kPvExact, 8, 2>(g2, st, p);
    else if (mode == kPvF16) launch_prefill<kPvF16, 8, 2>(g2, st, p);
    else launch_prefill<kPvGuard, 8, 2>(g2, st, p);
  } else {
    if (mode == kPvExact) launch_prefill<kPvExact, 8>(g, st, p);
    else if (mode == kPvF16) launch_prefill<kPvF16, 8>(g, st, p);
    else launch_prefill<kPvGuard, 8>(g, st, p);
  }
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
