// Host-side task-map builder ("Task Assign"): runs once per inference step, before the
// attention kernels of all layers ([P4] "腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级"
// §二.1; [P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案 steps 1-4).
//
// Plain C++17 with no HIP dependency: the same object is linked into liblbsa.so and can be
// built with g++ alone.  No allocation: every pass walks the units in place and writes into
// the caller's buffer.
//
// The fill never materialises the tile stream.  A cursor (unit, first unused tile) advances
// through the units; worker w consumes budget_w tiles, emitting one segment per unit it touches.
// Budgets follow [P2] "大模型推理性能优化新范式" §二.1: base = T / W, plus one for the first
// T % W workers.

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <functional>
#include <queue>
#include <utility>
#include <vector>

#include "lbsa.h"

namespace {

inline int64_t tiles_for(int64_t extent, int64_t tile) { return extent > 0 ? (extent + tile - 1) / tile : 0; }

// A unit source yields (b, q_tile_index, extent) in batch-major order.
struct DecodeUnits {
  const int32_t* lens;
  int32_t B;
  int64_t count() const { return B; }
  template <class F> bool each(F&& f) const {
    for (int32_t b = 0; b < B; ++b)
      if (!f(b, 0, (int64_t)lens[b])) return false;
    return true;
  }
};

struct PrefillUnits {
  const int32_t* q_lens;
  const int32_t* kv_lens;
  int32_t B;
  int32_t q_tile;
  bool causal;
  int64_t count() const {
    int64_t n = 0;
    for (int32_t b = 0; b < B; ++b) n += tiles_for(q_lens[b], q_tile);
    return n;
  }
  template <class F> bool each(F&& f) const {
    for (int32_t b = 0; b < B; ++b) {
      const int64_t ql = q_lens[b], kl = kv_lens[b];
      const int64_t blocks = tiles_for(ql, q_tile);
      for (int64_t i = 0; i < blocks; ++i) {
        const int64_t last_row_end = ql < (i + 1) * q_tile ? ql : (i + 1) * q_tile;
        const int64_t extent = causal ? kl - ql + last_row_end : kl;
        if (!f(b, (int32_t)i, extent)) return false;
      }
    }
    return true;
  }
};

struct Writer {
  int32_t* map;
  int32_t W, U;
  int64_t seg_base() const { return LBSA_MAP_HEADER_WORDS + (W + 1) + (U + 1) + 2 * (int64_t)U; }
  int32_t* worker_ptr() const { return map + LBSA_MAP_HEADER_WORDS; }
  int32_t* unit_ptr() const { return map + LBSA_MAP_HEADER_WORDS + W + 1; }
  int32_t* units() const { return map + LBSA_MAP_HEADER_WORDS + W + 1 + U + 1; }
  int32_t* seg(int64_t i) const { return map + seg_base() + 4 * i; }
};

// Greedy equal-budget fill.  With `w` null only the segment count is returned.
template <class Units>
int64_t fill(const Units& units, int64_t T, int32_t W, int64_t tile, const Writer* w) {
  const int64_t base = T / W, rem = T % W;
  int64_t segs = 0;
  int32_t worker = 0;
  int64_t left = W > 0 ? base + (0 < rem ? 1 : 0) : 0;  // budget left for `worker`
  if (w) w->worker_ptr()[0] = 0;
  // close every worker whose budget is exhausted (including zero budgets)
  auto advance_workers = [&]() {
    while (left == 0 && worker < W) {
      ++worker;
      if (w) w->worker_ptr()[worker] = (int32_t)segs;
      if (worker < W) left = base + (worker < rem ? 1 : 0);
    }
  };
  advance_workers();
  int64_t u = 0;
  units.each([&](int32_t b, int32_t qt, int64_t extent) {
    if (w) {
      w->unit_ptr()[u] = (int32_t)segs;
      w->units()[2 * u] = b;
      w->units()[2 * u + 1] = qt;
    }
    const int64_t n = tiles_for(extent, tile);
    int64_t t = 0;
    while (t < n) {
      if (worker >= W) return false;  // budgets sum to T, so this cannot happen
      const int64_t take = (n - t) < left ? (n - t) : left;
      if (w) {
        int32_t* s = w->seg(segs);
        const int64_t end = (t + take) * tile;
        s[0] = b;
        s[1] = qt;
        s[2] = (int32_t)(t * tile);
        s[3] = (int32_t)(end < extent ? end : extent);
      }
      ++segs;
      t += take;
      left -= take;
      advance_workers();
    }
    ++u;
    return true;
  });
  if (w) w->unit_ptr()[u] = (int32_t)segs;
  return segs;
}

template <class Units>
int plan_units(const Units& units, int32_t B, int32_t W, int32_t kv_tile, int32_t q_tile,
               int32_t* map, int32_t cap, int32_t* words_out) {
  // pass 1: U, T and validation
  int64_t U = 0, T = 0;
  bool ok = units.each([&](int32_t, int32_t, int64_t extent) {
    if (extent < 0) return false;
    ++U;
    T += tiles_for(extent, kv_tile);
    return T <= INT32_MAX && extent <= INT32_MAX;
  });
  if (!ok || U > INT32_MAX / 4) return LBSA_ERR_INVALID;
  // pass 2: S
  Writer probe{nullptr, W, (int32_t)U};
  const int64_t S = fill(units, T, W, kv_tile, nullptr);
  const int64_t words = probe.seg_base() + 4 * S;
  if (words > INT32_MAX) return LBSA_ERR_INVALID;
  if (words_out) *words_out = (int32_t)words;
  if (words > cap) return LBSA_ERR_CAPACITY;
  // pass 3: write
  Writer wr{map, W, (int32_t)U};
  map[0] = LBSA_MAP_VERSION;
  map[1] = B;
  map[2] = W;
  map[3] = kv_tile;
  map[4] = (int32_t)S;
  map[5] = (int32_t)T;
  map[6] = q_tile;
  map[7] = (int32_t)U;
  const int64_t S2 = fill(units, T, W, kv_tile, &wr);
  return S2 == S ? LBSA_OK : LBSA_ERR_INVALID;
}

// Cost-weighted contiguous fill (a comparison planner): the stream of attn_plan, with tile costs in
// KV tokens (as [P5] "大模型推理性能优化揭秘" §五(一) sizes its tiles) plus split_cost on each
// request's first tile.  Tile i goes to worker floor(W (2 P_i + c_i) / (2 C)) — P_i the cost before
// it, C the total — so workers take contiguous stretches whose costs are within one tile's cost of
// C / W.  One walk over the tiles per pass, no allocation; the map is version 1.
//
// With per-worker rates (attn_plan_rated) worker w's share of the cost line is [C R_w / R, C R_(w+1) / R)
// (R_w the rates of the workers before w, R their total) and tile i goes to the last worker whose
// share starts at or before its midpoint: 2 C R_w <= R (2 P_i + c_i).  The midpoints increase along
// the stream, so the worker index only moves forward; zero-rate workers are stepped over.
int64_t weighted_fill(const int32_t* lens, int32_t B, int32_t W, int64_t tile, int64_t split_cost, int64_t C,
                      const Writer* wr, const int32_t* rates = nullptr, int64_t R = 0) {
  int64_t segs = 0, before = 0;
  int32_t w_rated = 0;       // current worker of the rated walk
  int64_t share_next = 0;    // R_(w_rated + 1)
  if (rates) share_next = rates[0];
  int32_t w_open = 0;   // workers <= w_open have their worker_ptr set
  bool have = false;
  int32_t run_b = 0, run_w = 0;
  int64_t run_t0 = 0, run_t1 = 0;
  auto close = [&]() {
    if (!have) return;
    if (wr) {
      int32_t* sg = wr->seg(segs);
      const int64_t end = (run_t1 + 1) * tile;
      sg[0] = run_b;
      sg[1] = 0;
      sg[2] = (int32_t)(run_t0 * tile);
      sg[3] = (int32_t)(end < lens[run_b] ? end : lens[run_b]);
    }
    ++segs;
    have = false;
  };
  if (wr) wr->worker_ptr()[0] = 0;
  for (int32_t b = 0; b < B; ++b) {
    close();
    if (wr) {
      wr->unit_ptr()[b] = (int32_t)segs;
      wr->units()[2 * b] = b;
      wr->units()[2 * b + 1] = 0;
    }
    const int64_t L = lens[b];
    const int64_t n = tiles_for(L, tile);
    for (int64_t t = 0; t < n; ++t) {
      const int64_t c = (L - t * tile < tile ? L - t * tile : tile) + (t == 0 ? split_cost : 0);
      int32_t w;
      if (rates) {
        const __int128 mid2 = (__int128)R * (2 * before + c);
        while (w_rated + 1 < W && 2 * (__int128)C * share_next <= mid2) share_next += rates[++w_rated];
        w = w_rated;
      } else {
        w = (int32_t)((__int128)W * (2 * before + c) / (2 * (__int128)C));
      }
      before += c;
      if (have && w != run_w) close();
      if (have) {
        run_t1 = t;
        continue;
      }
      for (; w_open < w; ++w_open)
        if (wr) wr->worker_ptr()[w_open + 1] = (int32_t)segs;
      have = true;
      run_b = b;
      run_w = w;
      run_t0 = run_t1 = t;
    }
  }
  close();
  if (wr) {
    wr->unit_ptr()[B] = (int32_t)segs;
    for (; w_open < W; ++w_open) wr->worker_ptr()[w_open + 1] = (int32_t)segs;
  }
  return segs;
}
}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case LBSA_OK: return "ok";
    case LBSA_ERR_INVALID: return "invalid argument";
    case LBSA_ERR_CAPACITY: return "map buffer too small";
    case LBSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LBSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t attn_map_words(int32_t num_units, int32_t num_workers, int64_t total_tiles_upper) {
  if (num_units < 0 || num_workers < 0 || total_tiles_upper < 0) return -1;
  int64_t s_max = (int64_t)num_workers + num_units - 1;
  if (total_tiles_upper < s_max) s_max = total_tiles_upper;
  if (s_max < 0) s_max = 0;
  const int64_t words = LBSA_MAP_HEADER_WORDS + (int64_t)num_workers + 1 + num_units + 1 +
                        2 * (int64_t)num_units + 4 * s_max;
  return words > INT32_MAX ? -1 : (int32_t)words;
}

int attn_plan(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile,
              int32_t* map, int32_t map_capacity, int32_t* map_words_out) {
  if (B < 0 || num_workers < 1 || tile < 1 || !map || map_capacity < 0) return LBSA_ERR_INVALID;
  if (B > 0 && !seq_lens) return LBSA_ERR_INVALID;
  DecodeUnits units{seq_lens, B};
  return plan_units(units, B, num_workers, tile, 1, map, map_capacity, map_words_out);
}

int attn_plan_prefill(const int32_t* q_lens, const int32_t* kv_lens, int32_t B,
                      int32_t num_workers, int32_t q_tile, int32_t kv_tile, int32_t causal,
                      int32_t* map, int32_t map_capacity, int32_t* map_words_out) {
  if (B < 0 || num_workers < 1 || q_tile < 1 || kv_tile < 1 || !map || map_capacity < 0)
    return LBSA_ERR_INVALID;
  if (B > 0 && (!q_lens || !kv_lens)) return LBSA_ERR_INVALID;
  for (int32_t b = 0; b < B; ++b)
    if (q_lens[b] < 0 || kv_lens[b] < 0 || q_lens[b] > kv_lens[b]) return LBSA_ERR_INVALID;
  PrefillUnits units{q_lens, kv_lens, B, q_tile, causal != 0};
  return plan_units(units, B, num_workers, kv_tile, q_tile, map, map_capacity, map_words_out);
}

int attn_plan_static(const int32_t* seq_lens, int32_t B, int32_t num_splits, int32_t tile,
                     int32_t* map, int32_t map_capacity, int32_t* map_words_out) {
  if (B < 0 || num_splits < 1 || tile < 1 || !map || map_capacity < 0) return LBSA_ERR_INVALID;
  if (B > 0 && !seq_lens) return LBSA_ERR_INVALID;
  int64_t T = 0, Wp = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_lens[b] < 0) return LBSA_ERR_INVALID;
    const int64_t n = tiles_for(seq_lens[b], tile);
    T += n;
    Wp += n < num_splits ? n : num_splits;
  }
  if (T > INT32_MAX) return LBSA_ERR_INVALID;
  const int64_t U = B, S = Wp;
  const int64_t words = LBSA_MAP_HEADER_WORDS + (Wp + 1) + (U + 1) + 2 * U + 4 * S;
  if (words > INT32_MAX) return LBSA_ERR_INVALID;
  if (map_words_out) *map_words_out = (int32_t)words;
  if (words > map_capacity) return LBSA_ERR_CAPACITY;
  Writer wr{map, (int32_t)Wp, (int32_t)U};
  map[0] = LBSA_MAP_VERSION;
  map[1] = B;
  map[2] = (int32_t)Wp;
  map[3] = tile;
  map[4] = (int32_t)S;
  map[5] = (int32_t)T;
  map[6] = 1;
  map[7] = (int32_t)U;
  int64_t s = 0;
  wr.worker_ptr()[0] = 0;
  for (int32_t b = 0; b < B; ++b) {
    wr.unit_ptr()[b] = (int32_t)s;
    wr.units()[2 * b] = b;
    wr.units()[2 * b + 1] = 0;
    const int64_t L = seq_lens[b];
    const int64_t n = tiles_for(L, tile);
    const int64_t k = n < num_splits ? n : num_splits;
    int64_t t0 = 0;
    for (int64_t c = 0; c < k; ++c) {
      const int64_t size = n / k + (c < n % k ? 1 : 0);
      int32_t* seg = wr.seg(s);
      const int64_t end = (t0 + size) * tile;
      seg[0] = b;
      seg[1] = 0;
      seg[2] = (int32_t)(t0 * tile);
      seg[3] = (int32_t)(end < L ? end : L);
      t0 += size;
      ++s;
      wr.worker_ptr()[s] = (int32_t)s;
    }
  }
  wr.unit_ptr()[B] = (int32_t)s;
  return LBSA_OK;
}

int attn_plan_weighted(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile, int32_t split_cost,
                       int32_t* map, int32_t map_capacity, int32_t* map_words_out) {
  if (B < 0 || num_workers < 1 || tile < 1 || split_cost < 0 || !map || map_capacity < 0) return LBSA_ERR_INVALID;
  if (B > 0 && !seq_lens) return LBSA_ERR_INVALID;
  int64_t T = 0, C = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_lens[b] < 0) return LBSA_ERR_INVALID;
    T += tiles_for(seq_lens[b], tile);
    C += (int64_t)seq_lens[b] + (seq_lens[b] > 0 ? split_cost : 0);   // widened before the sum
  }
  if (T > INT32_MAX) return LBSA_ERR_INVALID;
  Writer probe{nullptr, num_workers, B};
  const int64_t S = weighted_fill(seq_lens, B, num_workers, tile, split_cost, C, nullptr);
  const int64_t words = probe.seg_base() + 4 * S;
  if (words > INT32_MAX) return LBSA_ERR_INVALID;
  if (map_words_out) *map_words_out = (int32_t)words;
  if (words > map_capacity) return LBSA_ERR_CAPACITY;
  Writer wr{map, num_workers, B};
  map[0] = LBSA_MAP_VERSION;
  map[1] = B;
  map[2] = num_workers;
  map[3] = tile;
  map[4] = (int32_t)S;
  map[5] = (int32_t)T;
  map[6] = 1;
  map[7] = B;
  return weighted_fill(seq_lens, B, num_workers, tile, split_cost, C, &wr) == S ? LBSA_OK : LBSA_ERR_INVALID;
}

int attn_plan_rated(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile, int32_t split_cost,
                    const int32_t* worker_rates, int32_t* map, int32_t map_capacity, int32_t* map_words_out) {
  if (B < 0 || num_workers < 1 || tile < 1 || split_cost < 0 || !worker_rates || !map || map_capacity < 0)
    return LBSA_ERR_INVALID;
  if (B > 0 && !seq_lens) return LBSA_ERR_INVALID;
  int64_t R = 0;
  for (int32_t w = 0; w < num_workers; ++w) {
    if (worker_rates[w] < 0 || worker_rates[w] > LBSA_RATE_MAX) return LBSA_ERR_INVALID;
    R += worker_rates[w];
  }
  if (R == 0) return LBSA_ERR_INVALID;
  int64_t T = 0, C = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_lens[b] < 0) return LBSA_ERR_INVALID;
    T += tiles_for(seq_lens[b], tile);
    C += (int64_t)seq_lens[b] + (seq_lens[b] > 0 ? split_cost : 0);
  }
  if (T > INT32_MAX) return LBSA_ERR_INVALID;
  Writer probe{nullptr, num_workers, B};
  const int64_t S = weighted_fill(seq_lens, B, num_workers, tile, split_cost, C, nullptr, worker_rates, R);
  const int64_t words = probe.seg_base() + 4 * S;
  if (words > INT32_MAX) return LBSA_ERR_INVALID;
  if (map_words_out) *map_words_out = (int32_t)words;
  if (words > map_capacity) return LBSA_ERR_CAPACITY;
  Writer wr{map, num_workers, B};
  map[0] = LBSA_MAP_VERSION_PLACED;
  map[1] = B;
  map[2] = num_workers;
  map[3] = tile;
  map[4] = (int32_t)S;
  map[5] = (int32_t)T;
  map[6] = 1;
  map[7] = B;
  return weighted_fill(seq_lens, B, num_workers, tile, split_cost, C, &wr, worker_rates, R) == S ? LBSA_OK
                                                                                                  : LBSA_ERR_INVALID;
}

// LPT bucket packing ([P5] "大模型推理性能优化揭秘：从算子到系统的全链路技术解析" §五(一)), the
// comparison planner: tiles in decreasing token size (ties in stream order), each onto the worker
// with the smallest token load (ties to the lowest index).  Unlike the contiguous fill it needs
// O(T) host memory (the tile list and a heap), so it is not meant for the per-step hot path.
int attn_plan_lpt(const int32_t* seq_lens, int32_t B, int32_t num_workers, int32_t tile,
                  int32_t* map, int32_t map_capacity, int32_t* map_words_out) {
  if (B < 0 || num_workers < 1 || tile < 1 || !map || map_capacity < 0) return LBSA_ERR_INVALID;
  if (B > 0 && !seq_lens) return LBSA_ERR_INVALID;
  int64_t T = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_lens[b] < 0) return LBSA_ERR_INVALID;
    T += tiles_for(seq_lens[b], tile);
  }
  if (T > INT32_MAX) return LBSA_ERR_INVALID;
  struct Piece {
    int32_t size, b, t;
  };
  std::vector<Piece> pieces;
  pieces.reserve((size_t)T);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = tiles_for(seq_lens[b], tile);
    for (int64_t t = 0; t < n; ++t) {
      const int64_t left = (int64_t)seq_lens[b] - t * tile;
      pieces.push_back({(int32_t)(left < tile ? left : tile), b, (int32_t)t});
    }
  }
  std::stable_sort(pieces.begin(), pieces.end(), [](const Piece& x, const Piece& y) { return x.size > y.size; });
  // least-loaded worker: min-heap on (load, worker index)
  using Slot = std::pair<int64_t, int32_t>;
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
  for (int32_t w = 0; w < num_workers; ++w) heap.push({0, w});
  std::vector<int32_t> owner(pieces.size());
  for (size_t i = 0; i < pieces.size(); ++i) {
    Slot s = heap.top();
    heap.pop();
    owner[i] = s.second;
    s.first += pieces[i].size;
    heap.push(s);
  }
  // per worker, its tiles in stream order; consecutive tiles of one request form one segment
  struct Run {
    int32_t w, b, t0, t1;
  };
  std::vector<int32_t> idx(pieces.size());
  for (size_t i = 0; i < idx.size(); ++i) idx[i] = (int32_t)i;
  std::sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
    if (owner[x] != owner[y]) return owner[x] < owner[y];
    if (pieces[x].b != pieces[y].b) return pieces[x].b < pieces[y].b;
    return pieces[x].t < pieces[y].t;
  });
  std::vector<Run> runs;
  for (int32_t i : idx) {
    const Piece& p = pieces[i];
    if (!runs.empty() && runs.back().w == owner[i] && runs.back().b == p.b && runs.back().t1 == p.t - 1)
      runs.back().t1 = p.t;
    else
      runs.push_back({owner[i], p.b, p.t, p.t});
  }
  const int64_t S = (int64_t)runs.size();
  const int64_t words = LBSA_MAP_HEADER_WORDS + (int64_t)num_workers + 1 + (int64_t)B + 1 + 2 * (int64_t)B +
                        4 * S + S;
  if (words > INT32_MAX) return LBSA_ERR_INVALID;
  if (map_words_out) *map_words_out = (int32_t)words;
  if (words > map_capacity) return LBSA_ERR_CAPACITY;
  // slots: segments in unit-major order (request, then first tile)
  std::vector<int32_t> by_unit(runs.size());
  for (size_t i = 0; i < by_unit.size(); ++i) by_unit[i] = (int32_t)i;
  std::sort(by_unit.begin(), by_unit.end(), [&](int32_t x, int32_t y) {
    if (runs[x].b != runs[y].b) return runs[x].b < runs[y].b;
    return runs[x].t0 < runs[y].t0;
  });
  std::vector<int32_t> slot_of(runs.size());
  for (size_t k = 0; k < by_unit.size(); ++k) slot_of[by_unit[k]] = (int32_t)k;
  Writer wr{map, num_workers, B};
  map[0] = LBSA_MAP_VERSION_ORDERED;
  map[1] = B;
  map[2] = num_workers;
  map[3] = tile;
  map[4] = (int32_t)S;
  map[5] = (int32_t)T;
  map[6] = 1;
  map[7] = B;
  // unit table and unit_ptr
  {
    int64_t k = 0;
    for (int32_t b = 0; b < B; ++b) {
      wr.unit_ptr()[b] = (int32_t)k;
      wr.units()[2 * b] = b;
      wr.units()[2 * b + 1] = 0;
      while (k < S && runs[by_unit[k]].b == b) ++k;
    }
    wr.unit_ptr()[B] = (int32_t)S;
  }
  for (int64_t k = 0; k < S; ++k) {
    const Run& r = runs[by_unit[k]];
    int32_t* sg = wr.seg(k);
    const int64_t end = ((int64_t)r.t1 + 1) * tile;
    sg[0] = r.b;
    sg[1] = 0;
    sg[2] = (int32_t)((int64_t)r.t0 * tile);
    sg[3] = (int32_t)(end < seq_lens[r.b] ? end : seq_lens[r.b]);
  }
  // worker_ptr and the order list (runs are already worker-major, stream order inside a worker)
  int32_t* order = wr.seg(S);
  int64_t k = 0;
  for (int32_t w = 0; w < num_workers; ++w) {
    wr.worker_ptr()[w] = (int32_t)k;
    while (k < S && runs[k].w == w) {
      order[k] = slot_of[k];
      ++k;
    }
  }
  wr.worker_ptr()[num_workers] = (int32_t)S;
  return LBSA_OK;
}

}  // extern "C"
