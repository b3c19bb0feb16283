// Device-side task-map builder: the decode work map of attn_plan, built on the GPU from device-resident
// lengths, bit for bit the same buffer.
//
// The pages build the map once per inference step before the attention of every layer ([P4]
// "腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级" §二.1; [P3] "Hy3 Preview AI Infra 推理优化精读笔记"
// §3.1 方案 steps 1-4).  Building it on the device keeps a serving step free of host round trips:
// the lengths never leave the GPU, and plan + split-KV + combine can be captured in one HIP graph
// and replayed with new lengths.
//
// One workgroup of 1024 threads.  The greedy contiguous fill has a closed form: with T tiles and W
// workers, base = T / W and rem = T % W, worker w owns stream tiles [start_w, start_w + budget_w)
// with start_w = w * base + min(w, rem), and the worker of stream tile t is
//   t / (base + 1)                             if t < rem * (base + 1)
//   rem + (t - rem * (base + 1)) / base        otherwise.
// A request whose tiles are [pre_b, pre_b + n_b) of the stream therefore has one segment per worker
// from worker(pre_b) to worker(pre_b + n_b - 1); its segments are consecutive in the map, so
// unit_ptr is the exclusive prefix sum of these spans.  A worker's segment count is the number of
// non-empty requests its tile range touches (two binary searches over pre and a prefix count of
// non-empty requests).  Scans are block-wide; per-request prefix values are kept in the map's
// unit[] area while the map is built and overwritten with (b, 0) at the end.

#include <climits>

#include "common.h"
#include "lbsa.h"

namespace lbsa {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// Exclusive prefix sum of v over the workgroup; *total gets the sum of all v.  Every thread calls it.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* total, int64_t* lds /* [kPlanWaves + 1] */) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int64_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t up = __shfl_up(incl, d, 64);
    if (lane >= d) incl += up;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t acc = 0;
    for (int i = 0; i < kPlanWaves; ++i) {
      const int64_t t = lds[i];
      lds[i] = acc;
      acc += t;
    }
    lds[kPlanWaves] = acc;
  }
  __syncthreads();
  const int64_t excl = lds[wave] + incl - v;
  *total = lds[kPlanWaves];
  __syncthreads();   // lds is reused by the next call
  return excl;
}

__global__ __launch_bounds__(kPlanThreads) void plan_device_kernel(const int32_t* __restrict__ lens, int32_t B,
                                                                  int32_t W, int32_t tile, int32_t* __restrict__ map,
                                                                  int32_t cap) {
  __shared__ int64_t scan_lds[kPlanWaves + 1];
  __shared__ int32_t bad_lds;
  const int tid = threadIdx.x;
  int32_t* worker_ptr = map + LBSA_MAP_HEADER_WORDS;
  int32_t* unit_ptr = worker_ptr + W + 1;
  int32_t* units = unit_ptr + B + 1;   // [B][2]; while the map is built: (nonempty-before count, pre)
  int32_t* segs = units + 2 * (int64_t)B;
  if (tid == 0) bad_lds = 0;
  __syncthreads();

  auto tiles = [&](int64_t L) -> int64_t { return L > 0 ? (L + tile - 1) / tile : 0; };

  // pass A: pre_b (exclusive prefix of tile counts) and the count of non-empty requests before b
  int64_t T = 0, NZ = 0;
  for (int64_t b0 = 0; b0 < B; b0 += kPlanThreads) {
    const int64_t b = b0 + tid;
    const int64_t L = b < B ? lens[b] : 0;
    if (L < 0) bad_lds = 1;
    const int64_t n = tiles(L);
    int64_t tot, nz_tot;
    const int64_t pre = T + block_exclusive_scan(n, &tot, scan_lds);
    const int64_t nzb = NZ + block_exclusive_scan(n > 0 ? 1 : 0, &nz_tot, scan_lds);
    if (b < B) {
      units[2 * b] = (int32_t)nzb;
      units[2 * b + 1] = (int32_t)(pre < INT32_MAX ? pre : INT32_MAX);
    }
    T += tot;
    NZ += nz_tot;
  }
  __syncthreads();
  if (bad_lds || T > INT32_MAX) {
    if (tid == 0) map[0] = LBSA_ERR_INVALID;
    return;
  }
  const int64_t base = T / W, rem = T % W;
  const int64_t split = rem * (base + 1);
  auto worker_of = [&](int64_t t) -> int64_t { return t < split ? t / (base + 1) : rem + (t - split) / base; };
  auto start_of = [&](int64_t w) -> int64_t { return w * base + (w < rem ? w : rem); };
  // index of the last request whose pre is <= t (the request holding stream tile t, for t < T)
  auto holder = [&](int64_t t) -> int64_t {
    int64_t lo = 0, hi = B;   // first index with pre > t lies in [lo, hi]
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if ((int64_t)units[2 * mid + 1] <= t) lo = mid + 1; else hi = mid;
    }
    return lo - 1;
  };

  // pass B: span of every request (workers it touches) -> unit_ptr, S
  int64_t S = 0;
  for (int64_t b0 = 0; b0 < B; b0 += kPlanThreads) {
    const int64_t b = b0 + tid;
    int64_t span = 0;
    if (b < B) {
      const int64_t n = tiles(lens[b]);
      if (n > 0) {
        const int64_t pre = units[2 * b + 1];
        span = worker_of(pre + n - 1) - worker_of(pre) + 1;
      }
    }
    int64_t tot;
    const int64_t up = S + block_exclusive_scan(span, &tot, scan_lds);
    if (b < B) unit_ptr[b] = (int32_t)up;
    S += tot;
  }
  const int64_t words = LBSA_MAP_HEADER_WORDS + (int64_t)W + 1 + (int64_t)B + 1 + 2 * (int64_t)B + 4 * S;
  if (words > cap) {
    __syncthreads();
    if (tid == 0) {
      map[0] = LBSA_ERR_CAPACITY;
      map[4] = (int32_t)(S < INT32_MAX ? S : INT32_MAX);
    }
    return;
  }
  if (tid == 0) unit_ptr[B] = (int32_t)S;

  // pass C: segments per worker -> worker_ptr
  int64_t acc = 0;
  for (int64_t w0 = 0; w0 < W; w0 += kPlanThreads) {
    const int64_t w = w0 + tid;
    int64_t cnt = 0;
    if (w < W) {
      const int64_t start = start_of(w);
      const int64_t budget = base + (w < rem ? 1 : 0);
      if (budget > 0) {
        const int64_t fb = holder(start);
        const int64_t lb = holder(start + budget - 1);
        cnt = (int64_t)units[2 * lb] - units[2 * fb] + 1;
      }
    }
    int64_t tot;
    const int64_t wp = acc + block_exclusive_scan(cnt, &tot, scan_lds);
    if (w < W) worker_ptr[w] = (int32_t)wp;
    acc += tot;
  }
  if (tid == 0) worker_ptr[W] = (int32_t)S;

  // pass D: the segments, request by request (consecutive indices from unit_ptr[b])
  for (int64_t b = tid; b < B; b += kPlanThreads) {
    const int64_t L = lens[b];
    const int64_t n = tiles(L);
    if (n == 0) continue;
    const int64_t pre = units[2 * b + 1];
    const int64_t w_first = worker_of(pre);
    const int64_t w_last = worker_of(pre + n - 1);
    int64_t idx = unit_ptr[b];
    for (int64_t w = w_first; w <= w_last; ++w, ++idx) {
      const int64_t start = start_of(w);
      const int64_t end = start + base + (w < rem ? 1 : 0);
      const int64_t a = start > pre ? start : pre;
      const int64_t e = end < pre + n ? end : pre + n;
      const int64_t kv_end = (e - pre) * tile;
      int32_t* s = segs + 4 * idx;
      s[0] = (int32_t)b;
      s[1] = 0;
      s[2] = (int32_t)((a - pre) * tile);
      s[3] = (int32_t)(kv_end < L ? kv_end : L);
    }
  }
  __syncthreads();

  // pass E: the unit table proper, then the header
  for (int64_t b = tid; b < B; b += kPlanThreads) {
    units[2 * b] = (int32_t)b;
    units[2 * b + 1] = 0;
  }
  if (tid == 0) {
    map[1] = B;
    map[2] = W;
    map[3] = tile;
    map[4] = (int32_t)S;
    map[5] = (int32_t)T;
    map[6] = 1;
    map[7] = B;
    map[0] = LBSA_MAP_VERSION;
  }
}

}  // namespace lbsa

extern "C" int attn_plan_device(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile,
                                int32_t* map, int32_t map_capacity, void* stream) {
  if (B < 0 || num_workers < 1 || tile < 1 || !map || map_capacity < 0) return LBSA_ERR_INVALID;
  if (B > 0 && !seq_lens) return LBSA_ERR_INVALID;
  const int64_t fixed = LBSA_MAP_HEADER_WORDS + (int64_t)num_workers + 1 + (int64_t)B + 1 + 2 * (int64_t)B;
  if (fixed > INT32_MAX) return LBSA_ERR_INVALID;
  if (fixed > map_capacity) return LBSA_ERR_CAPACITY;
  hipLaunchKernelGGL(lbsa::plan_device_kernel, dim3(1), dim3(lbsa::kPlanThreads), 0,
                     static_cast<hipStream_t>(stream), seq_lens, B, num_workers, tile, map, map_capacity);
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
