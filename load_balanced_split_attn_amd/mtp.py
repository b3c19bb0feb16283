"""Multi-token decode (the verify step of multi-token prediction): plan once, run for every layer.

A multi-token-prediction step checks a few drafted tokens per request at once ([P3] "Hy3 Preview AI
Infra 推理优化精读笔记" §7), so each request carries q_len (1..4) query tokens: the last q_len
positions of its context, causal among themselves.  Every request is one planner unit of R =
max q_len rows whose KV tiles the greedy equal-budget fill spreads over workers exactly as in
decode ([P3] §3.1 方案); the decode kernel runs the rows x 8 query heads of a KV head as MFMA
columns, so the KV stream is read once for all rows.
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (KV_BF16, KV_FP8_E4M3, attn_combine, attn_plan_prefill, attn_query_workers, attn_splitkv_mtp,
               map_header, max_splits_of)
from .decode import choose_list_major, device_map

MAX_ROWS = 4


class MtpDecodeStep:
    def __init__(self, q_lens: Sequence[int], kv_lens: Sequence[int], device, num_workers: Optional[int] = None,
                 tile: int = 512, head_groups: int = 8, kv_dtype: int = KV_BF16, num_q_heads: int = 64,
                 head_dim: int = 128, launch_order: str = "auto"):
        """launch_order as in ``decode.DecodeStep``: list-major when the per-XCD token totals of the
        map's lists are within 1% ("auto"), or as asked; the partials are the same either way."""
        device = torch.device(device)
        self.q_lens_host = [int(x) for x in q_lens]
        self.kv_lens_host = [int(x) for x in kv_lens]
        if any(q < 0 or q > MAX_ROWS for q in self.q_lens_host):
            raise ValueError(f"multi-token decode takes 0..{MAX_ROWS} query tokens per request")
        if any(q > k for q, k in zip(self.q_lens_host, self.kv_lens_host)):
            raise ValueError("a request's query tokens are part of its context: q_len <= kv_len")
        self.R = max([1] + self.q_lens_host)
        if num_workers is None:
            num_workers = attn_query_workers(device.index or 0, head_groups, kv_dtype)
        self.map_host = attn_plan_prefill(self.q_lens_host, self.kv_lens_host, num_workers, self.R, tile, True)
        hdr = map_header(self.map_host)
        self.W, self.S, self.U, self.T = hdr["W"], hdr["S"], hdr["U"], hdr["T"]
        self.max_splits = max_splits_of(self.map_host)
        self.head_groups = head_groups
        self.kv_dtype = kv_dtype
        self.device = device
        self.list_major = choose_list_major(self.map_host, head_groups, launch_order)
        self.map = device_map(self.map_host, self.list_major, device)
        self.q_lens = torch.tensor(self.q_lens_host, dtype=torch.int32, device=device)
        self.kv_lens = torch.tensor(self.kv_lens_host, dtype=torch.int32, device=device)
        starts = [0]
        for n in self.q_lens_host[:-1]:
            starts.append(starts[-1] + n)
        self.rows = sum(self.q_lens_host)
        self.q_start = torch.tensor(starts[:len(self.q_lens_host)], dtype=torch.int32, device=device)
        S = max(self.S, 1)
        self.part_m = torch.empty((S, self.R, num_q_heads), dtype=torch.float32, device=device)
        self.part_l = torch.empty((S, self.R, num_q_heads), dtype=torch.float32, device=device)
        self.part_o = torch.empty((S, self.R, num_q_heads, head_dim), dtype=torch.float32, device=device)

    def splitkv(self, q, k_cache, v_cache, block_table, scale: float, kv_scales=None, stream=None) -> None:
        if (k_cache.dtype == torch.uint8) != (self.kv_dtype == KV_FP8_E4M3):
            raise ValueError("cache dtype does not match the kv_dtype this step was planned for")
        attn_splitkv_mtp(q, k_cache, v_cache, block_table, self.q_lens, self.q_start, self.kv_lens, self.map,
                         self.W, self.S, self.head_groups, self.R, scale, self.part_m, self.part_l, self.part_o,
                         kv_scales=kv_scales, stream=stream)

    def combine(self, out, stream=None) -> None:
        attn_combine(self.part_m, self.part_l, self.part_o, self.map, self.U, out, rows_per_unit=self.R,
                     q_lens=self.q_lens, q_start=self.q_start, max_splits=self.max_splits, stream=stream)

    def __call__(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 scale: Optional[float] = None, out: Optional[torch.Tensor] = None, kv_scales=None,
                 stream=None) -> torch.Tensor:
        if scale is None:
            scale = q.shape[-1] ** -0.5
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        self.splitkv(q, k_cache, v_cache, block_table, scale, kv_scales=kv_scales, stream=stream)
        self.combine(out, stream=stream)
        return out
