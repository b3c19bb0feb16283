"""Chunked prefill over a cached prefix: plan once, run for every layer.

Prefill units are 256-row (or 128-row) blocks of each request's query chunk; their 512-token KV tiles are packed
onto workers by the same greedy equal-budget planner as decode ([P3] "Hy3 Preview AI Infra 推理优化
精读笔记" §3.1 方案), then the split-KV kernel and the combine kernel run on the current stream.
P.V precision (exact_pv): None (default) runs fp16 P.V on checked chunks of V, falling back to
bf16 V for a chunk fp16 does not hold exactly; True always bf16 V with hi + lo P; False the
unchecked fp16 path, exact only for V = 0 and 2^-17 <= |V| <= 65504.
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import attn_combine, attn_plan_prefill, attn_splitkv_prefill, map_header, max_splits_of

Q_TILE = 256   # rows per unit: eight waves of 32 rows share each staged K/V chunk (128: two heads per workgroup)


class PrefillStep:
    def __init__(self, q_lens: Sequence[int], kv_lens: Sequence[int], device, num_workers: int = 128,
                 kv_tile: int = 512, causal: bool = True, num_q_heads: int = 64, head_dim: int = 128,
                 exact_pv: Optional[bool] = None, q_tile: int = Q_TILE):
        device = torch.device(device)
        self.q_lens_host = [int(x) for x in q_lens]
        self.kv_lens_host = [int(x) for x in kv_lens]
        self.causal = bool(causal)
        self.exact_pv = None if exact_pv is None else bool(exact_pv)
        if q_tile not in (128, 256):
            raise ValueError("q_tile must be 128 or 256 (32 rows per wave, 4 or 8 waves per query head)")
        self.q_tile = q_tile
        self.map_host = attn_plan_prefill(self.q_lens_host, self.kv_lens_host, num_workers, q_tile, kv_tile,
                                          self.causal)
        hdr = map_header(self.map_host)
        self.W, self.S, self.U, self.T = hdr["W"], hdr["S"], hdr["U"], hdr["T"]
        self.max_splits = max_splits_of(self.map_host)
        self.device = device
        self.map = torch.from_numpy(self.map_host).to(device)
        self.q_lens = torch.tensor(self.q_lens_host, dtype=torch.int32, device=device)
        self.kv_lens = torch.tensor(self.kv_lens_host, dtype=torch.int32, device=device)
        starts = [0]
        for n in self.q_lens_host[:-1]:
            starts.append(starts[-1] + n)
        self.rows = sum(self.q_lens_host)
        self.q_start = torch.tensor(starts[:len(self.q_lens_host)], dtype=torch.int32, device=device)
        S = max(self.S, 1)
        self.part_m = torch.empty((S, q_tile, num_q_heads), dtype=torch.float32, device=device)
        self.part_l = torch.empty((S, q_tile, num_q_heads), dtype=torch.float32, device=device)
        self.part_o = torch.empty((S, q_tile, num_q_heads, head_dim), dtype=torch.float32, device=device)

    def splitkv(self, q, k_cache, v_cache, block_table, scale: float, stream=None) -> None:
        attn_splitkv_prefill(q, k_cache, v_cache, block_table, self.q_lens, self.q_start, self.kv_lens, self.map,
                             self.W, self.S, scale, self.part_m, self.part_l, self.part_o, causal=self.causal,
                             q_tile=self.q_tile, exact_pv=self.exact_pv, stream=stream)

    def combine(self, out, stream=None) -> None:
        attn_combine(self.part_m, self.part_l, self.part_o, self.map, self.U, out, rows_per_unit=self.q_tile,
                     q_lens=self.q_lens, q_start=self.q_start, max_splits=self.max_splits, stream=stream)

    def __call__(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 scale: Optional[float] = None, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        if scale is None:
            scale = q.shape[-1] ** -0.5
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        self.splitkv(q, k_cache, v_cache, block_table, scale, stream=stream)
        self.combine(out, stream=stream)
        return out
