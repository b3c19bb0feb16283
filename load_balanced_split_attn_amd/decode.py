"""Decode attention for one inference step: plan once, run for every layer.

The pages build the task map once per inference step and let the attention kernel of every layer
read it ([P4] "腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级" §二.1; [P3] "Hy3 Preview AI
Infra 推理优化精读笔记" §3.1 方案 step 4).  ``DecodeStep`` does that: the constructor calls the
host planner and copies the map to the device once; each call launches the split-KV kernel and the
combine kernel on the current stream, reusing the map and the partial buffers.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

from . import (KV_BF16, KV_FP8_E4M3, MAP_VERSION_PLACED, attn_combine, attn_plan, attn_plan_lpt, attn_plan_rated,
               attn_plan_static, attn_plan_weighted, attn_query_workers,
               attn_splitkv, attn_splitkv_claimed, attn_splitkv_fp8, map_header, max_splits_of)

XCDS = 8   # accelerator complex dies; the dispatcher places workgroup b on XCD b mod 8
LIST_MAJOR_BALANCE = 1.01   # largest per-XCD token max/mean at which "auto" launches list-major


def list_tokens(map_host: np.ndarray) -> np.ndarray:
    """KV tokens of each worker's list in a host work map (versions 1-3)."""
    hdr = map_header(map_host)
    W, U = hdr["W"], hdr["U"]
    wptr = np.asarray(map_host[8:8 + W + 1], dtype=np.int64)
    segs = np.asarray(map_host[8 + (W + 1) + (U + 1) + 2 * U:], dtype=np.int64)[:4 * hdr["S"]].reshape(-1, 4)
    if hdr["version"] == 2:
        order = np.asarray(map_host[8 + (W + 1) + (U + 1) + 2 * U + 4 * hdr["S"]:], dtype=np.int64)
        segs = segs[order[:hdr["S"]]]
    seg_tokens = np.maximum(segs[:, 3] - segs[:, 2], 0)
    return np.array([seg_tokens[wptr[w]:wptr[w + 1]].sum() for w in range(W)], dtype=np.float64)


def xcd_token_balance(map_host: np.ndarray) -> float:
    """Largest over mean of the per-XCD token totals when list w runs on XCD w mod 8 (1.0 for a map
    with no tokens)."""
    tok = list_tokens(map_host)
    per_xcd = np.array([tok[x::XCDS].sum() for x in range(XCDS)])
    return float(per_xcd.max() / per_xcd.mean()) if per_xcd.mean() > 0 else 1.0


def choose_list_major(map_host: np.ndarray, head_groups: int, launch_order: str = "auto",
                      claiming: bool = False) -> bool:
    """Whether a step's split-KV launch runs the map list-major (see ``DecodeStep``'s launch_order):
    always for a version-3 map; for a version-1 map with more than one head group and W a multiple of
    8 when asked ("list") or when its per-XCD token totals are within 1% ("auto"); never otherwise
    (a run-time claiming launch takes its order from its counter)."""
    if launch_order not in ("auto", "head", "list"):
        raise ValueError(f"unknown launch_order {launch_order!r} (auto, head or list)")
    hdr = map_header(map_host)
    if hdr["version"] == MAP_VERSION_PLACED:
        return True
    if hdr["version"] != 1 or head_groups <= 1 or hdr["W"] % XCDS or claiming:
        return False
    return launch_order == "list" or (launch_order == "auto" and xcd_token_balance(map_host) <= LIST_MAJOR_BALANCE)


def device_map(map_host: np.ndarray, list_major: bool, device) -> torch.Tensor:
    """The map's device copy; a version-1 map launched list-major carries the version-3 word there
    (the host map is left as planned)."""
    words = map_host.copy()
    if list_major:
        words[0] = MAP_VERSION_PLACED
    return torch.from_numpy(words).to(device)


class DecodeStep:
    def __init__(self, seq_lens: Sequence[int], device, num_workers: Optional[int] = None, tile: int = 512,
                 head_groups: int = 8, num_q_heads: int = 64, head_dim: int = 128,
                 static_splits: Optional[int] = None, kv_dtype: int = KV_BF16, planner: str = "greedy",
                 split_cost: int = 0, resident_workgroups: Optional[int] = None,
                 xcd_rates: Optional[Sequence[int]] = None, launch_order: str = "auto"):
        """resident_workgroups: run the split-KV kernel with run-time claiming (that many one-wave
        workgroups take the map's (list, KV head) items from a device counter) instead of one
        workgroup per (list, head group); needs head_groups equal to the KV head count.
        planner "rated": attn_plan_rated with worker w's rate xcd_rates[w mod 8] (the XCD its
        workgroups run on in the map's list-major order; see ``calibrate_xcd_rates``).
        launch_order: the order in which the split-KV launch runs a version-1 map's (list, head
        group) workgroups.  "head": workgroup b takes list b div G, head group b mod G, so every XCD
        runs one head group of every list and streams exactly the same tokens.  "list": workgroup b
        takes list b mod W, head group b div W, so all of list w's workgroups run on XCD w mod 8 and
        stream its pages' heads together (requested by writing the version-3 word into the device
        copy of the map; the host map stays as planned).  "auto": list-major when the head groups
        are more than one, W is a multiple of 8 and the per-XCD token totals under it are within 1%
        of each other (``xcd_token_balance``): it measured 0.4-1.3% faster on such batches and up to
        1.6% slower where whole lists leave the XCDs 2% apart.  The partials are the same either way."""
        device = torch.device(device)
        self.seq_lens_host = [int(x) for x in seq_lens]
        if static_splits is not None:
            self.map_host = attn_plan_static(self.seq_lens_host, static_splits, tile)
        else:
            if num_workers is None:
                num_workers = attn_query_workers(device.index or 0, head_groups, kv_dtype)
            if planner == "greedy":
                self.map_host = attn_plan(self.seq_lens_host, num_workers, tile)
            elif planner == "lpt":
                self.map_host = attn_plan_lpt(self.seq_lens_host, num_workers, tile)
            elif planner == "weighted":
                self.map_host = attn_plan_weighted(self.seq_lens_host, num_workers, tile, split_cost)
            elif planner == "rated":
                if xcd_rates is None or len(xcd_rates) != XCDS:
                    raise ValueError("planner 'rated' needs xcd_rates, one rate per XCD")
                rates = [int(xcd_rates[w % XCDS]) for w in range(num_workers)]
                self.map_host = attn_plan_rated(self.seq_lens_host, num_workers, rates, tile, split_cost)
            else:
                raise ValueError(f"unknown planner {planner!r} (greedy, lpt, weighted or rated)")
        hdr = map_header(self.map_host)
        self.W, self.S, self.U, self.T = hdr["W"], hdr["S"], hdr["U"], hdr["T"]
        self.max_splits = max_splits_of(self.map_host)
        self.tile = tile
        self.head_groups = head_groups
        self.kv_dtype = kv_dtype
        self.device = device
        self.list_major = choose_list_major(self.map_host, head_groups, launch_order,
                                            claiming=resident_workgroups is not None)
        self.map = device_map(self.map_host, self.list_major, device)
        self.seq_lens = torch.tensor(self.seq_lens_host, dtype=torch.int32, device=device)
        S = max(self.S, 1)
        self.part_m = torch.empty((S, num_q_heads), dtype=torch.float32, device=device)
        self.part_l = torch.empty((S, num_q_heads), dtype=torch.float32, device=device)
        self.part_o = torch.empty((S, num_q_heads, head_dim), dtype=torch.float32, device=device)
        self.resident = resident_workgroups
        self.claim_state = torch.zeros(2, dtype=torch.int32, device=device) if resident_workgroups else None

    def splitkv(self, q, k_cache, v_cache, block_table, scale: float, timing=None, stream=None,
                kv_scales=None) -> None:
        """bf16 cache, or (kv_dtype KV_FP8_E4M3) uint8 codes with kv_scales = (k_scale, v_scale)."""
        if self.resident:
            attn_splitkv_claimed(q, k_cache, v_cache, block_table, self.seq_lens, self.map, self.W, self.S,
                                 self.resident, self.claim_state, scale, self.part_m, self.part_l, self.part_o,
                                 kv_scales=kv_scales if self.kv_dtype == KV_FP8_E4M3 else None, timing=timing,
                                 stream=stream)
            return
        if self.kv_dtype == KV_FP8_E4M3:
            if kv_scales is None:
                raise ValueError("an 8-bit cache needs kv_scales=(k_scale, v_scale)")
            attn_splitkv_fp8(q, k_cache, v_cache, kv_scales[0], kv_scales[1], block_table, self.seq_lens, self.map,
                             self.W, self.S, self.head_groups, scale, self.part_m, self.part_l, self.part_o,
                             timing=timing, stream=stream)
        else:
            attn_splitkv(q, k_cache, v_cache, block_table, self.seq_lens, self.map, self.W, self.S,
                         self.head_groups, scale, self.part_m, self.part_l, self.part_o, timing=timing,
                         stream=stream)

    def combine(self, out, stream=None) -> None:
        attn_combine(self.part_m, self.part_l, self.part_o, self.map, self.U, out, max_splits=self.max_splits,
                     stream=stream)

    def __call__(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 scale: Optional[float] = None, out: Optional[torch.Tensor] = None, timing=None,
                 stream=None, kv_scales=None) -> torch.Tensor:
        if scale is None:
            scale = q.shape[-1] ** -0.5
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        self.splitkv(q, k_cache, v_cache, block_table, scale, timing=timing, stream=stream, kv_scales=kv_scales)
        self.combine(out, stream=stream)
        return out


def xcd_rates_from_timing(timing: torch.Tensor, map_host: np.ndarray, head_groups: int,
                          scale_to: int = 1 << 16, list_major: Optional[bool] = None) -> List[int]:
    """Per-XCD streaming rates from one or more instrumented split-KV launches over ``map_host``
    (``timing`` rows as the kernel writes them: start, end, HW_ID, XCC_ID per workgroup; several
    launches stacked along the first axis): on each XCD, the KV tokens its workgroups streamed over
    the sum of their durations.  Scaled so the fastest XCD has ``scale_to``.  ``list_major``: the
    order the launches ran in (default: the map's own, list-major for version 3)."""
    t = timing.cpu().numpy().astype(np.int64).reshape(-1, 4)
    hdr = map_header(map_host)
    W = hdr["W"]
    tokens = list_tokens(map_host)
    if list_major is None:
        list_major = hdr["version"] == MAP_VERSION_PLACED
    per_launch = W * head_groups
    b = np.arange(t.shape[0]) % per_launch
    w = b % W if list_major else b // head_groups
    xcc = t[:, 3] & 0xF
    dur = (t[:, 1] - t[:, 0]).astype(np.float64)
    rate = np.zeros(XCDS)
    for x in range(XCDS):
        sel = xcc == x
        if dur[sel].sum() <= 0:
            raise ValueError(f"no timed workgroup ran on XCD {x}")
        rate[x] = tokens[w[sel]].sum() / dur[sel].sum()
    return [max(1, int(round(scale_to * r / rate.max()))) for r in rate]


def calibrate_xcd_rates(step: "DecodeStep", q, k_cache, v_cache, block_table, scale: float, launches: int = 3,
                        kv_scales=None) -> List[int]:
    """Run ``step``'s split-KV launch ``launches`` times with the kernel's timestamps on (after one
    untimed launch) and return the per-XCD rates of ``xcd_rates_from_timing``: the input of
    ``DecodeStep(..., planner="rated", xcd_rates=...)``.  Each XCD's rate is its tokens over its
    workgroups' time, whichever order the step launches in."""
    if step.resident:
        raise ValueError("calibrate on a static launch (no run-time claiming)")
    step.splitkv(q, k_cache, v_cache, block_table, scale, kv_scales=kv_scales)
    n = step.W * step.head_groups
    timing = torch.zeros((launches, n, 4), dtype=torch.int64, device=step.device)
    for i in range(launches):
        step.splitkv(q, k_cache, v_cache, block_table, scale, timing=timing[i], kv_scales=kv_scales)
    torch.cuda.synchronize(step.device)
    return xcd_rates_from_timing(timing, step.map_host, step.head_groups, list_major=step.list_major)


class DeviceDecodeStep:
    """Decode with the work map built on the device.

    The lengths stay on the GPU (``seq_lens``, int32[B]; update them in place), and ``plan``,
    ``splitkv`` and ``combine`` are stream-ordered kernel launches with no host synchronisation,
    so a whole step can be captured in one HIP graph and replayed with new lengths.  Buffers are
    sized for the worst case: the map for S <= W + B - 1 segments, the partials likewise.
    """

    def __init__(self, batch: int, device, num_workers: Optional[int] = None, tile: int = 512,
                 head_groups: int = 8, kv_dtype: int = KV_BF16, num_q_heads: int = 64, head_dim: int = 128):
        from . import attn_plan_device, device_map_words
        self._plan_device = attn_plan_device
        device = torch.device(device)
        if num_workers is None:
            num_workers = attn_query_workers(device.index or 0, head_groups, kv_dtype)
        self.B, self.W, self.tile = int(batch), int(num_workers), int(tile)
        self.head_groups = head_groups
        self.kv_dtype = kv_dtype
        self.device = device
        self.map = torch.zeros(device_map_words(self.B, self.W), dtype=torch.int32, device=device)
        self.seq_lens = torch.zeros(self.B, dtype=torch.int32, device=device)
        self.S_max = max(1, self.W + self.B - 1)
        self.part_m = torch.empty((self.S_max, num_q_heads), dtype=torch.float32, device=device)
        self.part_l = torch.empty((self.S_max, num_q_heads), dtype=torch.float32, device=device)
        self.part_o = torch.empty((self.S_max, num_q_heads, head_dim), dtype=torch.float32, device=device)

    def plan(self, stream=None) -> None:
        self._plan_device(self.seq_lens, self.W, self.tile, self.map, stream=stream)

    def splitkv(self, q, k_cache, v_cache, block_table, scale: float, timing=None, stream=None,
                kv_scales=None) -> None:
        if self.kv_dtype == KV_FP8_E4M3:
            if kv_scales is None:
                raise ValueError("an 8-bit cache needs kv_scales=(k_scale, v_scale)")
            attn_splitkv_fp8(q, k_cache, v_cache, kv_scales[0], kv_scales[1], block_table, self.seq_lens, self.map,
                             self.W, self.S_max, self.head_groups, scale, self.part_m, self.part_l, self.part_o,
                             timing=timing, stream=stream)
        else:
            attn_splitkv(q, k_cache, v_cache, block_table, self.seq_lens, self.map, self.W, self.S_max,
                         self.head_groups, scale, self.part_m, self.part_l, self.part_o, timing=timing,
                         stream=stream)

    def combine(self, out, stream=None) -> None:
        # the split count per request is only known on the device: pass the worker count as the bound
        attn_combine(self.part_m, self.part_l, self.part_o, self.map, self.B, out, max_splits=self.W, stream=stream)

    def __call__(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 scale: Optional[float] = None, out: Optional[torch.Tensor] = None, stream=None,
                 kv_scales=None) -> torch.Tensor:
        if scale is None:
            scale = q.shape[-1] ** -0.5
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        self.plan(stream=stream)
        self.splitkv(q, k_cache, v_cache, block_table, scale, stream=stream, kv_scales=kv_scales)
        self.combine(out, stream=stream)
        return out
