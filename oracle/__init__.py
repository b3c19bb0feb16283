"""CPU oracle for load-balanced split-KV attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports it and
shares no code with it: no kernels, headers, helpers, tables or constants.

Four parts:

* ``oracle.plan``      - the tile cut, the equal budgets and the greedy fill
  that build the work map, written out step by step.  Integer-only; the GPU
  library's planner must reproduce its int32 buffer bit for bit.
* ``oracle.attention`` - exact softmax attention in float64 (the plain
  definition), per-split partials (max, sum-exp, unnormalised output) and the
  combine that merges them.
* ``oracle.fp8``       - the value of an element of an 8-bit (OCP E4M3) KV
  cache with per-KV-head scales, and decode attention over such a cache
  (dequantise, then ``oracle.attention``).
* ``oracle.store_kv``  - the producer step of a decode step: RMSNorm, RoPE and
  Hadamard rotation of the new q/k, bf16 or E4M3 rounding, the values stored.

Sources (the web pages this method is described on):

* [P3] "Hy3 Preview AI Infra 推理优化精读笔记", §3.1 "Attention：动态切分和负载均衡"
  (问题 / 方案 / 收益), §2 model shape table, §14 glossary entry "Split-KV".
* [P4] "腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级", §二.1 "Attention：动态调度
  负载均衡，根治推理长尾延迟".
* [P1] pwwt.cn explainer of the same article, §3.1 "算子优化", paragraph on
  dynamically scheduled load-balanced attention.
* [P2] "大模型推理性能优化新范式：Hy3架构下的全栈优化技术拆解", §二.1, the
  ``dynamic_tile_scheduler`` pseudocode (budget arithmetic only).

Pins (what each function is checked against, outside itself) are listed in
``tests/test_oracle_*.py``.  Every function here is pinned; none is
"parity unpinned".  The exact segment placement inside the map follows the
reading stated in ``oracle.plan`` (the pages' placement figure is not in the
text); its pins are the worked example's tile and budget counts plus
invariants that any contiguous equal-budget fill must satisfy.
"""

from . import attention, fp8, plan, store_kv  # noqa: F401
