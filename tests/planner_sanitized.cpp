// Test driver for the host planners (csrc/plan.cpp), built by tests/test_planner_sanitized.py with
// g++ and the address and undefined-behaviour sanitizers.  One case per input line:
//
//   kind B p1 p2 p3 p4 short  arrays...
//
//   kind 0 attn_plan          p1 = workers, p2 = tile                       lens[B]
//   kind 1 attn_plan_static   p1 = splits,  p2 = tile                       lens[B]
//   kind 2 attn_plan_prefill  p1 = workers, p2 = q_tile, p3 = kv_tile, p4 = causal   q_lens[B] kv_lens[B]
//   kind 3 attn_plan_lpt      p1 = workers, p2 = tile                       lens[B]
//   kind 4 attn_plan_weighted p1 = workers, p2 = tile, p3 = split_cost      lens[B]
//
// The planner is first asked for its size (capacity 0), then called on a heap buffer of exactly
// that many words (short = 0) or one word fewer (short = 1, which must fail with the capacity
// status without writing past the buffer).  Output per case: "status words w0 w1 ...".

#include <cstdint>
#include <cstdio>
#include <iostream>
#include <vector>

#include "lbsa.h"

static int call(int kind, const std::vector<int32_t>& a, const std::vector<int32_t>& b, int32_t B, int32_t p1,
                int32_t p2, int32_t p3, int32_t p4, int32_t* map, int32_t cap, int32_t* need) {
  const int32_t* lens = B ? a.data() : nullptr;
  switch (kind) {
    case 0: return attn_plan(lens, B, p1, p2, map, cap, need);
    case 1: return attn_plan_static(lens, B, p1, p2, map, cap, need);
    case 2: return attn_plan_prefill(lens, B ? b.data() : nullptr, B, p1, p2, p3, p4, map, cap, need);
    case 3: return attn_plan_lpt(lens, B, p1, p2, map, cap, need);
    case 4: return attn_plan_weighted(lens, B, p1, p2, p3, map, cap, need);
    default: return -100;
  }
}

int main() {
  int kind;
  while (std::cin >> kind) {
    int64_t B, p1, p2, p3, p4, shortcap;
    std::cin >> B >> p1 >> p2 >> p3 >> p4 >> shortcap;
    std::vector<int32_t> a(B), b(kind == 2 ? B : 0);
    for (auto& x : a) std::cin >> x;
    for (auto& x : b) std::cin >> x;
    int32_t probe_word = 0, need = 0;
    int st = call(kind, a, b, (int32_t)B, (int32_t)p1, (int32_t)p2, (int32_t)p3, (int32_t)p4, &probe_word, 0, &need);
    if (st != LBSA_ERR_CAPACITY && st != LBSA_OK) {
      std::printf("%d 0\n", st);
      continue;
    }
    const int32_t cap = need - (int32_t)shortcap;
    std::vector<int32_t>* buf = new std::vector<int32_t>(cap > 0 ? cap : 1);
    int32_t words = 0;
    st = call(kind, a, b, (int32_t)B, (int32_t)p1, (int32_t)p2, (int32_t)p3, (int32_t)p4, buf->data(), cap, &words);
    std::printf("%d %d", st, st == LBSA_OK ? words : 0);
    if (st == LBSA_OK)
      for (int32_t i = 0; i < words; ++i) std::printf(" %d", (*buf)[i]);
    std::printf("\n");
    delete buf;
  }
  return 0;
}
