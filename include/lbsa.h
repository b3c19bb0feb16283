/*
 * lbsa.h - load-balanced split-KV attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of liblbsa.so.  Only C types cross it: plain host or device pointers,
 * sizes and a HIP stream passed as void*.  The library never allocates device
 * memory, never synchronises the device and keeps no state between calls other
 * than a cached occupancy query per device.
 *
 * The method (sources are web pages; cited by title and section):
 *   [P3] "Hy3 Preview AI Infra 推理优化精读笔记", §3.1 Attention：动态切分和负载均衡
 *        (问题 / 方案 / 收益), §2 model table, §14 glossary ("Split-KV", "Tile", "CTA").
 *   [P4] "腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级", §二.1 Attention.
 *   [P1] pwwt.cn explainer of the same article, §3.1 算子优化.
 *   [P2] "大模型推理性能优化新范式：Hy3架构下的全栈优化技术拆解", §二.1 (budget pseudocode).
 * Every request's KV range is cut into uniform tiles; the tiles of the whole
 * batch form one stream; each worker (a workgroup here, a CTA on the pages'
 * GPU) gets an equal or near-equal tile budget and is filled greedily from the
 * stream, so a long request spans several workers.  This task map is built
 * once per inference step and read by the attention kernel of every layer; each
 * split writes a partial result and a combine kernel merges them.
 *
 * Status codes: every entry point returns LBSA_OK (0) or a negative code.
 * Kernels are asynchronous on the given stream: a device-side fault surfaces at
 * the caller's next synchronisation, not in the return code.
 *
 * ---------------------------------------------------------------------------
 * Work map: one flat little-endian int32 buffer
 *
 *   [0] version (1; 2 and 3 below)           [1] B  (requests)     [2] W (workers)      [3] kv_tile
 *   [4] S (segments)   [5] T  (total tiles)  [6] q_tile (1 for decode)
 *   [7] U (query units: one per request in decode, one per q_tile rows in prefill)
 *   worker_ptr[W+1]    segments of worker w:  [worker_ptr[w], worker_ptr[w+1])
 *   unit_ptr[U+1]      segments of unit u:    [unit_ptr[u], unit_ptr[u+1])
 *   unit[U][2]         (b, q_tile_index)
 *   seg[S][4]          (b, q_tile_index, kv_begin, kv_end), KV token range, end exclusive
 *
 * Segment i is one split and owns partial slot i.  Segments are stored in task
 * stream order, which is both worker-major and unit-major.  Total words:
 * 8 + (W+1) + (U+1) + 2U + 4S.
 *
 * ---------------------------------------------------------------------------
 * Tensor layouts (device memory, all caller-owned)
 *
 *   q        bf16 [rows, Hq, D]: decode rows = B (one query per request);
 *                                prefill rows = sum of q_len_b, request b from row q_start[b]
 *   k_cache, v_cache  [num_pages, Hkv] blocks, one contiguous block per (page, KV head),
 *            stored in rows of 64 bytes (w = 64 / element bytes elements per row: 32 for
 *            bf16, 64 for 8-bit codes):
 *              k_cache block  [D / w][page_size][w]   dim tile, token, dim inside the tile
 *              v_cache block  [page_size / w][D][w]   token tile, dim, token inside the tile
 *            i.e. K is token-major and V dim-major ("V transposed") inside 64-byte tiles; the
 *            kernels' load instructions then cover whole 128-byte lines.  Element (token t,
 *            dim d) of a block: K at ((d / w) * page_size + t) * w + d % w, V at
 *            ((t / w) * D + d) * w + t % w (in elements).
 *   block_table int32 [B, block_table_stride]: physical page of logical page p of request b
 *   part_m, part_l fp32 [S, R, Hq];  part_o fp32 [S, R, Hq, D]   (R = 1 decode, q_tile prefill)
 *   out      fp32 or bf16 [rows, Hq, D]
 * Query head h reads KV head h / (Hq / Hkv) (grouped-query attention; [P3] §2:
 * 64 query heads, 8 KV heads, head dim 128).
 * Partial (m, l, o) of a split: m = max scaled score (natural-log units),
 * l = sum exp(s - m), o = sum exp(s - m) v, not divided by l.  A split with no
 * visible key writes (-inf, 0, 0).
 */
#ifndef LBSA_H
#define LBSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LBSA_OK 0
#define LBSA_ERR_INVALID (-1)     /* null pointer, negative size, bad shape or alignment      */
#define LBSA_ERR_CAPACITY (-2)    /* map buffer too small; *map_words_out holds the size needed */
#define LBSA_ERR_UNSUPPORTED (-3) /* a shape the kernels are not built for (see each call)     */
#define LBSA_ERR_HIP (-4)         /* HIP runtime error at launch                              */
/* the same codes under the attn_ prefix of the entry points */
#define ATTN_OK LBSA_OK
#define ATTN_ERR_INVALID LBSA_ERR_INVALID
#define ATTN_ERR_CAPACITY LBSA_ERR_CAPACITY
#define ATTN_ERR_UNSUPPORTED LBSA_ERR_UNSUPPORTED
#define ATTN_ERR_HIP LBSA_ERR_HIP

#define LBSA_MAP_VERSION 1
#define LBSA_MAP_HEADER_WORDS 8

/* Human-readable name of a status code.  Never returns NULL. */
const char* attn_status_string(int status);

/*
 * Upper bound on the words of a map with U units, W workers and at most T tiles:
 * 8 + (W+1) + (U+1) + 2U + 4*min(T, W+U-1).  Returns -1 if an argument is negative
 * or the bound does not fit in int32.
 */
int32_t attn_map_words(int32_t num_units, int32_t num_workers, int64_t total_tiles_upper);

/*
 * Dynamic (load-balanced) decode work map ([P3] §3.1 方案 steps 1-4; [P2] budget
 * rule: base = T / W, the first T % W workers get one more tile).
 *   seq_lens      host int32[B], KV length of each request (>= 0); the single query of
 *                 request b sits at position seq_lens[b]-1 and sees keys [0, seq_lens[b])
 *   num_workers   W >= 1 work lists (one per worker; a worker may be run by several
 *                 workgroups, one per KV-head group)
 *   tile          tile size in KV tokens (>= 1; 512 in the pages' worked example)
 *   map           host int32[map_capacity], written with the layout above
 *   map_words_out optional (may be NULL): words written, or words needed on
 *                 LBSA_ERR_CAPACITY
 * Tile counts are ceilings; the stream is in batch order with tiles ascending;
 * worker w takes the next budget_w tiles; consecutive tiles of one request inside
 * one worker form one segment.  Pure host function: reentrant, deterministic,
 * allocation-free.  Errors: LBSA_ERR_INVALID (null pointer, B < 0, W < 1,
 * tile < 1, negative length, T beyond int32), LBSA_ERR_CAPACITY.
 */
int attn_plan(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile,
              int32_t* map, int32_t map_capacity, int32_t* map_words_out);

/*
 * The attn_plan map built on the device, for serving loops whose lengths live on the GPU and for
 * capture in a HIP graph together with the attention launches (the pages build the map once per
 * step before every layer's attention, [P4] §二.1; [P3] §3.1 方案 steps 1-4).  One workgroup
 * writes, on `stream`, exactly the buffer attn_plan writes for the same lengths.
 *   seq_lens      device int32[B]
 *   map           device int32[map_capacity]; attn_map_words(B, W, INT64_MAX) words always
 *                 suffice (S <= W + B - 1)
 * Host-side errors (returned): LBSA_ERR_INVALID (B < 0, W < 1, tile < 1, NULL pointers),
 * LBSA_ERR_CAPACITY (capacity below the map's fixed part, 8 + W+1 + B+1 + 2B words), LBSA_ERR_HIP.
 * Data errors are written to the device map instead, since the lengths are only known there:
 * map[0] = LBSA_MAP_VERSION on success, LBSA_ERR_INVALID for a negative length or more than
 * INT32_MAX tiles, LBSA_ERR_CAPACITY (with map[4] = the segment count needed) when the segments do
 * not fit.  Split and combine kernels given a map whose map[0] is not a map version (1, or 2 where
 * accepted) do nothing.
 */
int attn_plan_device(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile,
                     int32_t* map, int32_t map_capacity, void* stream);

/*
 * Cost-weighted contiguous fill, a comparison planner: the tile cut and task stream of attn_plan
 * ([P3] §3.1 方案 steps 1-2), with the equal budgets of steps 3-4 counted in cost instead of
 * tiles — a tile costs its KV tokens (the tile sizes of [P5] §五(一)) and a request's first tile
 * costs split_cost more (the fixed work of a split: query load, pipeline start, partial and
 * combine).  With P_i the cost of the stream before tile i, c_i its cost and C the total, tile i
 * goes to worker floor(W (2 P_i + c_i) / (2 C)): every worker takes one contiguous stretch of the
 * stream whose cost is within the largest tile cost of C / W.  Writes a version-1 map (the layout
 * of attn_plan, read by the same kernels), S <= W + B - 1.
 *   split_cost   >= 0, in KV tokens
 * O(B + T) time, no allocation.  Errors and capacity reporting as attn_plan (LBSA_ERR_INVALID also
 * for a negative split_cost).
 */
int attn_plan_weighted(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile,
                       int32_t split_cost, int32_t* map, int32_t map_capacity, int32_t* map_words_out);

/*
 * Rate-proportional contiguous fill: attn_plan_weighted's stream and tile costs, with worker w's
 * share of the cost line proportional to worker_rates[w] instead of equal.  The pages' scheduler
 * ([P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案 steps 3-4) gives every worker the same
 * budget, which equalises finish times when the workers stream at one rate; on a device whose
 * workgroups stream at different rates depending on where they run, equal finish times need budgets
 * in proportion to the rates.  With R_w the sum of the rates of workers 0 .. w-1 and R their total,
 * tile i (cost c_i, P_i the cost before it) goes to the last worker w with 2 C R_w <= R (2 P_i + c_i):
 * the worker whose share [C R_w / R, C R_(w+1) / R) holds the tile's midpoint.  A worker of rate 0
 * gets nothing; equal rates give attn_plan_weighted's lists exactly.
 *   worker_rates  host int32[num_workers], each in [0, LBSA_RATE_MAX], not all zero
 * The map is written in version 3 (LBSA_MAP_VERSION_PLACED): version 1's words, and the split-KV
 * launch (attn_splitkv, attn_splitkv_fp8) then runs workgroup b on list b mod W and
 * head group b div W, so with W a multiple of 8 every workgroup of list w runs on XCD w mod 8 (the
 * dispatcher places workgroup b on XCD b mod 8) and per-XCD rates can be given per worker.
 * attn_combine and the run-time claiming launch (whose order comes from its counter) accept it; the
 * prefill kernel takes version 1 only.  Any version-1 decode map may be launched in the same
 * list-major order by setting its word 0 to LBSA_MAP_VERSION_PLACED (its other words unchanged; the
 * partials are bitwise the same): that pays when the token totals of the lists on each XCD
 * (w mod 8) are nearly equal, and costs when they are not.  O(B + T + W) time, no allocation.  Errors and capacity reporting as attn_plan_weighted
 * (LBSA_ERR_INVALID also for a NULL worker_rates, a rate outside the range, or all rates zero).
 */
#define LBSA_MAP_VERSION_PLACED 3
#define LBSA_RATE_MAX (1 << 20)
int attn_plan_rated(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile, int32_t split_cost,
                    const int32_t* worker_rates, int32_t* map, int32_t map_capacity, int32_t* map_words_out);

/*
 * LPT comparison map ([P5] "大模型推理性能优化揭秘：从算子到系统的全链路技术解析" §五(一): tiles
 * sorted by decreasing size, each put on the least-loaded worker).  A tile's size and a worker's
 * load are counted in KV tokens; equal sizes keep stream order, equal loads go to the lowest worker
 * index; inside a worker the tiles run in stream order and consecutive tiles of one request merge
 * into one segment.  A request's tiles end up scattered over workers, so the map is written in
 * version 2 (LBSA_MAP_VERSION_ORDERED): segments unit-major (segment i = partial slot i), plus
 * order[S] after seg[S][4], and worker w runs segments order[worker_ptr[w] .. worker_ptr[w+1]).
 * attn_splitkv, attn_splitkv_fp8 and attn_combine accept it; the prefill and multi-token kernels take
 * version 1 only.  Uses O(T) host memory (not a per-step hot-path routine).  Arguments and errors as
 * attn_plan.
 */
#define LBSA_MAP_VERSION_ORDERED 2
int attn_plan_lpt(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile,
                  int32_t* map, int32_t map_capacity, int32_t* map_words_out);

/*
 * Static split-KV map, the imbalance baseline ([P3] §3.1 问题; [P4] §二.1: one
 * fixed split granularity for the whole batch).  Request b is cut into
 * k_b = min(num_splits, n_b) tile-aligned chunks whose tile counts differ by at
 * most one, larger chunks first; each chunk is its own worker with one segment,
 * so the map's W = sum_b k_b.  Arguments and errors as attn_plan.
 */
int attn_plan_static(const int32_t* seq_lens, int32_t B, int32_t num_splits, int32_t tile,
                     int32_t* map, int32_t map_capacity, int32_t* map_words_out);

/*
 * Prefill work map for chunked prefill over a cached prefix: request b has a
 * q_lens[b]-row query chunk that is the last q_lens[b] positions of a
 * kv_lens[b]-token context.  Units are (b, i) blocks of q_tile rows, batch-major;
 * under the causal mask unit (b, i) attends to keys
 * [0, kv_lens[b] - q_lens[b] + min(q_lens[b], (i+1)*q_tile)), otherwise to all
 * kv_lens[b] keys.  The units' kv_tile tiles are then filled exactly as in
 * attn_plan.  Errors as attn_plan, plus q_lens[b] > kv_lens[b] or q_tile < 1.
 */
int attn_plan_prefill(const int32_t* q_lens, const int32_t* kv_lens, int32_t B,
                      int32_t num_workers, int32_t q_tile, int32_t kv_tile, int32_t causal,
                      int32_t* map, int32_t map_capacity, int32_t* map_words_out);

/*
 * KV cache element types of the decode kernels.
 *   LBSA_KV_BF16      bf16 k_cache / v_cache (attn_splitkv)
 *   LBSA_KV_FP8_E4M3  8-bit OCP E4M3 codes with one fp32 scale per KV head for K and one for V
 *                     (attn_splitkv_fp8)
 */
#define LBSA_KV_BF16 0
#define LBSA_KV_FP8_E4M3 1

/*
 * Workers that fill the device with one resident wave of decode workgroups:
 * CUs x (resident split-KV workgroups per CU) / head_groups, for the decode kernel of cache type
 * kv_dtype (LBSA_KV_*) launched with head_groups workgroups per worker.  Cached per device and type;
 * safe to call from several host threads at once.
 * Errors: LBSA_ERR_INVALID (head_groups not a divisor of 8, unknown kv_dtype, device out of range),
 * LBSA_ERR_HIP.
 */
int attn_query_workers(int device, int32_t head_groups, int32_t kv_dtype, int32_t* num_workers_out);

/*
 * Split-KV decode kernel ([P3] §3.1 方案 step 4; [P4] §二.1): launches
 * num_workers x head_groups workgroups; workgroup (w, g) walks worker w's segment
 * list for the Hkv/head_groups KV heads of group g and writes one partial per
 * segment and query head.
 *   q, k_cache, v_cache, block_table  device, layouts above (16-byte aligned)
 *   num_pages     pages in the caches (physical page ids are clamped into range)
 *   seq_lens      device int32[B]; a segment's KV end is clamped to seq_lens[b]
 *   map           device copy of an attn_plan / attn_plan_static map for this batch
 *   num_workers, num_segments   W and S of that map (a map whose word 2 is not num_workers is
 *                 skipped on the device: nothing is written)
 *   head_groups   G, a divisor of Hkv
 *   part_m, part_l, part_o       device fp32 outputs sized by S (see layouts)
 *   timing        optional device uint64[W*G*4] (start, end, HW_ID, XCC_ID per
 *                 workgroup, device realtime clock); NULL disables recording
 *   stream        hipStream_t, or NULL for the null stream
 * Supported: head_dim 128, Hq/Hkv = 8, bf16, page_size a multiple of 64.
 * Errors: LBSA_ERR_INVALID, LBSA_ERR_UNSUPPORTED, LBSA_ERR_HIP.
 */
int attn_splitkv(const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                 const int32_t* seq_lens, const int32_t* map,
                 int32_t num_workers, int32_t num_segments, int32_t head_groups,
                 int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t page_size, float softmax_scale,
                 float* part_m, float* part_l, float* part_o,
                 uint64_t* timing, void* stream);

/*
 * Split-KV decode over an 8-bit KV cache (the 8-bit cache of the pages' production precision:
 * [P3] §1 and §14 "W8A8C8", §8 attention in FP8; [P4] §一: BF16 and FP8 formats).  Same work map,
 * launch shape, partial layout and errors as attn_splitkv; only the cache differs:
 *   k_cache, v_cache  uint8 OCP E4M3 codes in the blocked layout above (w = 64)
 *   k_scale, v_scale  device fp32[Hkv] (4-byte aligned): element x of KV head g stands for
 *                 e4m3(x) * k_scale[g] (keys) or e4m3(x) * v_scale[g] (values)
 * The codes are widened exactly to bf16 before the matrix products; q stays bf16.  Partials are in
 * real units (the scales are applied), so attn_combine merges them as usual.
 * Errors: as attn_splitkv, plus LBSA_ERR_INVALID for a missing or misaligned scale pointer.
 */
int attn_splitkv_fp8(const void* q, const void* k_cache, const void* v_cache,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                     const int32_t* seq_lens, const int32_t* map,
                     int32_t num_workers, int32_t num_segments, int32_t head_groups,
                     int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, float softmax_scale,
                     float* part_m, float* part_l, float* part_o,
                     uint64_t* timing, void* stream);

/*
 * Split-KV decode with run-time claiming of the map's lists ([P4] §二.1: the workers take their
 * tasks from the map at run time; [P3] §3.1 方案 step 4).  The map is attn_plan's (or attn_plan_static's,
 * attn_plan_weighted's, attn_plan_lpt's) for num_workers lists, typically several times the lists a
 * resident launch would get; instead of one workgroup per (list, KV head), resident_workgroups
 * workgroups of one wave each take items (list w, KV head g) in the order i = w * Hkv + g from a
 * device counter until every item is taken, so a list goes to whichever workgroup is free first.
 * Each item is run exactly once and writes the partial slots the static launch writes, with the
 * same arithmetic: the partials, and the attn_combine output, are bitwise those of attn_splitkv /
 * attn_splitkv_fp8 over the same map.
 *   kv_dtype      LBSA_KV_BF16 (k_scale, v_scale NULL) or LBSA_KV_FP8_E4M3 (scales as attn_splitkv_fp8)
 *   resident_workgroups  workgroups launched (>= 1; attn_query_workers(dev, 8, kv_dtype) * 8 fills
 *                 the device once)
 *   claim_state   device int32[2], 4-byte aligned, zero before the first launch; every launch
 *                 leaves it zero (the last workgroup to finish resets it).  Launches that share one
 *                 claim_state must not overlap (same stream, or ordered by events).
 *   timing        optional, device uint64[resident_workgroups * 4] (as attn_splitkv)
 * One wave per workgroup: head_groups is Hkv (every KV head its own item).  Other arguments, layouts
 * and errors as attn_splitkv; LBSA_ERR_INVALID also for a NULL or misaligned claim_state or
 * resident_workgroups < 1.
 */
int attn_splitkv_claimed(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                         const float* k_scale, const float* v_scale,
                         const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                         const int32_t* seq_lens, const int32_t* map, int32_t num_workers, int32_t num_segments,
                         int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, float softmax_scale, int32_t resident_workgroups,
                         int32_t* claim_state, float* part_m, float* part_l, float* part_o,
                         uint64_t* timing, void* stream);

/*
 * Multi-token decode (the verify step of multi-token prediction, [P3] §7: a step checks several
 * drafted tokens at once, so a request carries a few query tokens instead of one).  Request b has
 * q_lens[b] <= rows_per_unit query rows stored from row q_start[b] of q [rows, Hq, D]; they are the
 * last q_lens[b] positions of its kv_lens[b]-token context, and row j sees keys
 * [0, kv_lens[b] - q_lens[b] + j] (causal among the drafted tokens).  The map is
 * attn_plan_prefill(q_lens, kv_lens, W, q_tile = rows_per_unit, kv_tile, causal = 1), so every request
 * is one unit whose tiles the greedy fill spreads over workers exactly as in decode.  Launch shape
 * as attn_splitkv; each wave runs the rows x 8 query heads of its KV head as MFMA columns (up to 16
 * columns in one block for 2 rows, two blocks for 3 or 4), streaming K and V once for all rows.
 *   kv_dtype      LBSA_KV_BF16 (k_scale, v_scale NULL) or LBSA_KV_FP8_E4M3 (scales as attn_splitkv_fp8)
 *   q_lens, q_start, kv_lens  device int32[B]
 *   rows_per_unit R, 1..4 (the map's q_tile)
 *   part_m, part_l [S, R, Hq]; part_o [S, R, Hq, D]; rows j >= q_lens[b] of a slot are not written
 * Merge with attn_combine(..., rows_per_unit = R, q_lens, q_start, ...).
 * Errors: as attn_splitkv; LBSA_ERR_UNSUPPORTED for R > 4; LBSA_ERR_INVALID for a NULL
 * q_lens/q_start, an unknown kv_dtype or scales that do not match it.  Rows past R of a request
 * with q_lens[b] > R are not computed (the caller keeps q_lens[b] <= R).
 */
int attn_splitkv_mtp(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                     const int32_t* q_lens, const int32_t* q_start, const int32_t* kv_lens,
                     const int32_t* map, int32_t num_workers, int32_t num_segments, int32_t head_groups,
                     int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, int32_t rows_per_unit, float softmax_scale,
                     float* part_m, float* part_l, float* part_o, void* stream);

/*
 * Producer step of a decode step, fused ([P3] §4.1: RoPE, RMSNorm, Hadamard, quantisation and the
 * KV-cache write in one kernel; §8: q and k Hadamard-rotated before quantisation).  For each new
 * token b and head vector x (128 dims) of the projection output:
 *   1. RMSNorm if the gain is given: x / sqrt(mean(x^2) + norm_eps) * w (q_norm_w for q heads,
 *      k_norm_w for k heads; fp32[128] each, or NULL to skip)
 *   2. RoPE if rope_theta > 0, rotate-half: pairs (i, i + 64) turned by positions[b] * theta^(-i/64)
 *   3. Hadamard if hadamard = 1: x -> H x / sqrt(128), H the Sylvester-ordered Walsh-Hadamard matrix
 * q takes 1-3 and is written to q_out (bf16, round to nearest even; q_out may be q_in); k takes 1-3
 * and v none, and both are written at token positions[b] of request b's pages (block_table, the
 * blocked cache layout above), as bf16 (kv_dtype LBSA_KV_BF16) or as E4M3 codes of x / scale[head]
 * clamped to +-448, round to nearest even (LBSA_KV_FP8_E4M3, k_scale / v_scale fp32[Hkv]).
 *   q_in bf16 [B, Hq, 128]; k_in, v_in bf16 [B, Hkv, 128]; positions device int32[B]
 * A token whose position lies outside its block-table row, or whose page id is outside
 * [0, num_pages), is not stored (q_out is still written).  The caller advances seq_lens afterwards.
 * q_in, k_in, v_in, q_out and the caches must be 8-byte aligned, the gains 16-byte aligned.
 * Launches B x ceil((ceil(Hq/4) + 2 ceil(Hkv/4)) / 4) workgroups of 256 threads.
 * Errors: LBSA_ERR_INVALID (NULL pointers, negative sizes, eps or theta negative or NaN, hadamard
 * not 0/1, unknown kv_dtype, missing scales for E4M3, misaligned pointers), LBSA_ERR_UNSUPPORTED (head_dim != 128,
 * page_size not a multiple of 64), LBSA_ERR_HIP.
 */
int attn_store_kv(const void* q_in, const void* k_in, const void* v_in,
                  const float* q_norm_w, const float* k_norm_w, float norm_eps,
                  const int32_t* positions, float rope_theta, int32_t hadamard,
                  void* q_out, void* k_cache, void* v_cache, int32_t kv_dtype,
                  const float* k_scale, const float* v_scale,
                  const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                  int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t page_size, void* stream);

/*
 * Producer step of a prefill chunk: the same per-vector steps as attn_store_kv ([P3] §4.1), for a
 * chunk of consecutive new tokens per request (chunked prefill after a cached prefix, [P3] §6).
 * Request b appends q_lens[b] tokens: rows q_start[b] .. q_start[b] + q_lens[b] - 1 of q_in / k_in /
 * v_in / q_out, at positions positions[b] .. positions[b] + q_lens[b] - 1 of its pages.  q and k
 * take steps 1-3 per row exactly as attn_store_kv does; V is staged per 64-byte cache row (32 bf16
 * or 64 E4M3 tokens of one dim) so that every full row is written whole, and the rows the chunk
 * only partly covers keep the cache's bytes for the other tokens (the cached prefix before the
 * chunk, free slots after it).  The stored values are those of attn_store_kv token by token.
 *   q_lens, q_start, positions  device int32[B]; max_q_len >= every q_lens[b] (rows past it are not
 *                 processed); rows must lie inside q_in's [rows, Hq, 128] (not checked)
 *   other arguments as attn_store_kv; v_in and v_cache 16-byte aligned
 * A token at a position outside its block-table row, or in a page id outside [0, num_pages), is not
 * stored; a request with positions[b] < 0 stores nothing (its q rows are still written, rotated as
 * a token at position -1).
 * Launches B x max_q_len workgroups for q and k (one per row; its four waves take every fourth
 * group of four q or k heads) and B x (ceil(max_q_len / w) + 1) x Hkv for V (w = 32 bf16, 64 E4M3),
 * 256 threads each.
 * Errors: as attn_store_kv, plus LBSA_ERR_INVALID for NULL q_lens / q_start, max_q_len < 0 or a
 * grid beyond INT32_MAX workgroups.
 */
int attn_store_kv_chunk(const void* q_in, const void* k_in, const void* v_in,
                        const float* q_norm_w, const float* k_norm_w, float norm_eps,
                        const int32_t* q_lens, const int32_t* q_start, const int32_t* positions,
                        int32_t max_q_len, float rope_theta, int32_t hadamard,
                        void* q_out, void* k_cache, void* v_cache, int32_t kv_dtype,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                        int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t page_size, void* stream);

/*
 * KV-cache layout conversion between the token-major paged layout (each (page, KV head) block is
 * page_size rows of head_dim elements: a cache [num_pages, num_kv_heads, page_size, head_dim], the
 * layout most paged caches keep) and the blocked layout above that the attention kernels read.
 *   direction 0: src token-major -> dst blocked;  1: src blocked -> dst token-major
 *   kv_dtype  LBSA_KV_BF16 (2-byte elements) or LBSA_KV_FP8_E4M3 (1-byte codes, converted as bytes)
 *   src_k, src_v, dst_k, dst_v  device, 16-byte aligned, num_pages * num_kv_heads * page_size *
 *             head_dim elements each; dst must not overlap src (out of place)
 * Launches num_pages x num_kv_heads x page_size / 64 workgroups of 256 threads (one 64-token slice
 * of one block each: K as a permutation of 16-byte pieces, V transposed through LDS).
 * Errors: LBSA_ERR_INVALID (NULL or misaligned pointers, overlapping src and dst, unknown kv_dtype
 * or direction, negative sizes), LBSA_ERR_UNSUPPORTED (head_dim != 128, page_size not a multiple of
 * 64), LBSA_ERR_HIP.
 */
int attn_kv_layout(const void* src_k, const void* src_v, void* dst_k, void* dst_v, int32_t num_pages,
                   int32_t num_kv_heads, int32_t page_size, int32_t head_dim, int32_t kv_dtype,
                   int32_t direction, void* stream);

/*
 * Split-KV chunked-prefill kernel over a cached prefix (the greedy map of attn_plan_prefill
 * applied to prefill units; prefix reuse as in [P3] §6: a request's new chunk attends to its
 * cached prefix and, causally, to itself).  Request b has q_lens[b] query rows stored from row
 * q_start[b] of q [rows, Hq, D]; they are the last q_lens[b] positions of a kv_lens[b]-token
 * context held in the paged caches.  Launches 8 x ceil(W x Hkv / 8) x (q_tile / 32) workgroups of
 * eight waves: a workgroup walks worker w's segments for KV head g and 256 / q_tile of its query
 * heads (one for q_tile 256, two for 128), 32 rows of one head per wave.  Writes, for every segment
 * s and row i < q_tile of its unit that lies inside the chunk, part_m/part_l [S, q_tile, Hq] and
 * part_o [S, q_tile, Hq, D] (rows past the chunk are not written).  With causal != 0 row j sees
 * keys [0, kv_lens[b] - q_lens[b] + j]; otherwise all keys.
 *   q_lens, q_start, kv_lens  device int32[B]
 *   map           device copy of the attn_plan_prefill map (same q_tile, kv_tile % 64 == 0)
 *   flags         P.V precision.
 *                 0 (the default): V * 2^6 converted to fp16 while staged and P * 2^-6 rounded
 *                 to fp16 (11 significant bits; P below 2^-8 of the reference maximum in fp16's
 *                 subnormals, spacing 2^-18), with every staged V value checked: a 64-key chunk
 *                 holding a value outside 2^-23 <= |v| <= 1020 (where fp16 carries bf16 * 2^6
 *                 exactly; inf, NaN and exact zeros included) takes the exact path below instead,
 *                 so V is carried exactly for every bf16 input.
 *                 LBSA_PREFILL_EXACT_PV: V stays bf16 and P enters as bf16 hi + lo parts (~16
 *                 significant bits), for every chunk (~15-20% slower than 0 on N(0,1) inputs).
 *                 LBSA_PREFILL_F16_PV: the fp16 path with no check (~10% faster than 0).  The
 *                 conversion rounds toward zero, so V is carried exactly only where fp16 holds every
 *                 bf16 value: v = 0 and 2^-17 <= |v| <= 65504.  Below 2^-17 low bits are dropped
 *                 (fp16 subnormals, spacing 2^-24), below 2^-24 V becomes 0, above 65504 it
 *                 saturates to +-65504.  For V known to lie in that range only.
 * Supported: head_dim 128, Hq/Hkv = 8, bf16, q_tile 128 (workgroups of eight waves of 32 rows,
 * two query heads each) or 256 (eight waves, one query head), page_size a multiple of 64.  The map must come
 * from attn_plan_prefill with the same q_tile and num_workers (a map of another unit height or
 * worker count is skipped: nothing is written).
 * Errors: LBSA_ERR_INVALID (also unknown flag bits, or both precision flags), LBSA_ERR_UNSUPPORTED,
 * LBSA_ERR_HIP.
 */
#define LBSA_PREFILL_EXACT_PV 1
#define LBSA_PREFILL_F16_PV 2
int attn_splitkv_prefill(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                         const int32_t* q_lens, const int32_t* q_start, const int32_t* kv_lens,
                         const int32_t* map, int32_t num_workers, int32_t num_segments, int32_t B,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                         int32_t q_tile, int32_t causal, float softmax_scale,
                         float* part_m, float* part_l, float* part_o, int32_t flags, void* stream);

/*
 * Combine kernel ([P3] §3.1 方案 step 5): for every unit and query head merges the
 * unit's partial slots: M = max m_s, w_s = exp(m_s - M), out = sum w_s o_s / sum w_s l_s;
 * a unit without any visible key gets 0.
 *   map           device map (as given to the split kernel)
 *   num_units     U of the map
 *   rows_per_unit 1 for decode, q_tile for prefill
 *   q_lens, q_start  device int32[B] for prefill (row count and first output row of
 *                 request b); NULL for decode, where unit b writes output row b
 *   out_dtype     0 = fp32, 1 = bf16 (round to nearest even)
 *   max_splits    largest slot count of any unit (from the host map), or 0 if unknown; above 16 a
 *                 unit's slots are spread over four waves (a launch-shape hint, any value >= 0 is
 *                 correct)
 * Launch shapes: prefill with rows_per_unit >= 64 and 64 query heads takes one 256-thread
 * workgroup per (unit, row), each thread a quarter of one head (part_o and out then 16-byte
 * aligned, 8 for a bf16 out); otherwise one wave per (unit, row, query head) (part_o and out
 * 8-byte aligned, 4 for a bf16 out).
 * Errors: LBSA_ERR_INVALID (also a misaligned part_o or out), LBSA_ERR_UNSUPPORTED
 * (head_dim != 128), LBSA_ERR_HIP.
 */
int attn_combine(const float* part_m, const float* part_l, const float* part_o,
                 const int32_t* map, int32_t num_units, int32_t rows_per_unit,
                 const int32_t* q_lens, const int32_t* q_start,
                 int32_t num_q_heads, int32_t head_dim,
                 void* out, int32_t out_dtype, int32_t max_splits, void* stream);

/*
 * Allocation-free decode step, for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It is attn_splitkv (or, with
 * kv_dtype LBSA_KV_FP8_E4M3 and k_scale / v_scale, attn_splitkv_fp8) followed by attn_combine
 * (num_units = B, one row per unit) on `stream`, same arguments, layouts and kernels, except that
 * the partials live in a fixed array of the library, LBSA_NOALLOC_SCRATCH_BYTES of device memory
 * per GPU that the library holds from its first use on that GPU until the process ends.  The caller
 * passes inputs and `out` (fp32 or bf16 [B, Hq, D] by out_dtype, as attn_combine) only.
 *   The partials of a call need S * Hq * (D + 2) * 4 bytes (S = num_segments): up to 1,008
 *   segments at 64 query heads.  A larger call returns LBSA_ERR_CAPACITY and launches nothing.
 *   Nothing in the array has to start cleared: the split kernel writes every slot the combine
 *   reads in the same call.  Every call on one GPU shares that GPU's array: calls that may overlap
 *   on one GPU (on different streams, or from several host threads without ordering) race and must
 *   not be issued.
 * The call allocates nothing, host or device.  On the first call on a device it takes the array's
 * device address (hipGetSymbolAddress, with that device current); the device is the stream's
 * (hipStreamGetDevice), or the current one for a NULL stream.
 * Errors: as attn_splitkv / attn_splitkv_fp8 and attn_combine, plus LBSA_ERR_CAPACITY (above) and
 * LBSA_ERR_INVALID for an unknown kv_dtype or scales that do not match it.
 */
#define LBSA_NOALLOC_SCRATCH_BYTES (32u << 20)
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int32_t block_table_stride, int32_t num_pages,
                        const int32_t* seq_lens, const int32_t* map,
                        int32_t num_workers, int32_t num_segments, int32_t head_groups,
                        int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t page_size, float softmax_scale, int32_t max_splits,
                        void* out, int32_t out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LBSA_H */
