"""Load-balanced split-KV attention for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``liblbsa.so`` (C ABI declared in ``include/lbsa.h``).  The functions
here only marshal arguments: torch tensors supply device pointers and the current HIP stream,
every step of the path runs in the library (host planner in C++, kernels in HIP).  There is no
fallback: if the library is missing, the first call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "LbsaError", "lib", "attn_map_words", "attn_plan", "attn_plan_static", "attn_plan_prefill", "attn_plan_device",
    "attn_plan_lpt", "attn_plan_weighted", "attn_plan_rated", "MAP_VERSION_PLACED", "RATE_MAX",
    "attn_query_workers", "attn_splitkv", "attn_splitkv_fp8", "attn_splitkv_mtp", "attn_splitkv_prefill",
    "attn_combine", "attn_store_kv", "attn_store_kv_chunk", "attn_kv_layout", "attn_decode_noalloc", "attn_splitkv_claimed", "NOALLOC_SCRATCH_BYTES",
    "attn_status_string", "attn_probe_stream_read", "attn_probe_stream_read_rated", "attn_probe_mfma_rate", "map_header", "LIB_PATH", "KV_BF16", "KV_FP8_E4M3",
]

# cache element types (LBSA_KV_* in include/lbsa.h)
KV_BF16 = 0
KV_FP8_E4M3 = 1
# partial bytes attn_decode_noalloc holds per GPU (LBSA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20
# prefill P.V precision flags (LBSA_PREFILL_* in include/lbsa.h)
PREFILL_EXACT_PV = 1
PREFILL_F16_PV = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblbsa.so")

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_vp = ctypes.c_void_p
_c_i32 = ctypes.c_int32

_SIGNATURES = {
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_map_words": (ctypes.c_int32, [_c_i32, _c_i32, ctypes.c_int64]),
    "attn_plan": (ctypes.c_int, [_c_i32p, _c_i32, _c_i32, _c_i32, _c_i32p, _c_i32, _c_i32p]),
    "attn_plan_static": (ctypes.c_int, [_c_i32p, _c_i32, _c_i32, _c_i32, _c_i32p, _c_i32, _c_i32p]),
    "attn_plan_lpt": (ctypes.c_int, [_c_i32p, _c_i32, _c_i32, _c_i32, _c_i32p, _c_i32, _c_i32p]),
    "attn_plan_weighted": (ctypes.c_int, [_c_i32p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32p, _c_i32, _c_i32p]),
    "attn_plan_rated": (ctypes.c_int, [_c_i32p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32p, _c_i32p, _c_i32,
                                       _c_i32p]),
    "attn_plan_prefill": (ctypes.c_int, [_c_i32p, _c_i32p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                         _c_i32p, _c_i32, _c_i32p]),
    "attn_query_workers": (ctypes.c_int, [ctypes.c_int, _c_i32, _c_i32, _c_i32p]),
    "attn_plan_device": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_i32, _c_vp, _c_i32, _c_vp]),
    "attn_splitkv": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_vp,
                                    _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                    ctypes.c_float, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "attn_splitkv_fp8": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_vp,
                                        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                        ctypes.c_float, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "attn_splitkv_mtp": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp,
                                        _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                        _c_i32, _c_i32, _c_i32, ctypes.c_float, _c_vp, _c_vp, _c_vp, _c_vp]),
    "attn_store_kv": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_float, _c_vp, ctypes.c_float,
                                     _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32,
                                     _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp]),
    "attn_splitkv_claimed": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp,
                                            _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                            ctypes.c_float, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "attn_kv_layout": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                      _c_vp]),
    "attn_store_kv_chunk": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_float, _c_vp, _c_vp, _c_vp,
                                           _c_i32, ctypes.c_float, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_vp,
                                           _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp]),
    "attn_combine": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_vp,
                                    _c_i32, _c_i32, _c_vp, _c_i32, _c_i32, _c_vp]),
    "attn_probe_stream_read": (ctypes.c_int, [_c_vp, ctypes.c_int64, _c_i32, _c_vp, _c_vp]),
    "attn_probe_mfma_rate": (ctypes.c_int, [_c_i32, _c_i32, _c_vp, _c_vp]),
    "attn_probe_stream_read_rated": (ctypes.c_int, [_c_vp, ctypes.c_int64, _c_i32, _c_i32p, _c_vp, _c_vp]),
    "attn_decode_noalloc": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp,
                                           _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                           ctypes.c_float, _c_i32, _c_vp, _c_i32, _c_vp]),
    "attn_splitkv_prefill": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp,
                                            _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                            _c_i32, _c_i32, ctypes.c_float, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp]),
}

_lib = None


class LbsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load liblbsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m load_balanced_split_attn_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LbsaError(status, where)


def _i32_host(values: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(values, dtype=np.int64).astype(np.int32))


def _ptr_i32(a: np.ndarray):
    return a.ctypes.data_as(_c_i32p)


def attn_map_words(num_units: int, num_workers: int, total_tiles_upper: int) -> int:
    n = lib().attn_map_words(num_units, num_workers, total_tiles_upper)
    if n < 0:
        raise LbsaError(-1, "attn_map_words")
    return n


def _plan_call(fn, where, *args) -> np.ndarray:
    need = _c_i32(0)
    cap = 64
    while True:
        buf = np.zeros(cap, dtype=np.int32)
        st = fn(*args, _ptr_i32(buf), cap, ctypes.byref(need))
        if st == -2 and need.value > cap:
            cap = need.value
            continue
        _check(st, where)
        return buf[:need.value].copy()


def attn_plan(seq_lens: Sequence[int], num_workers: int, tile: int = 512) -> np.ndarray:
    """Dynamic work map (host int32 array)."""
    lens = _i32_host(seq_lens)
    return _plan_call(lib().attn_plan, "attn_plan", _ptr_i32(lens), len(lens), num_workers, tile)


def attn_plan_static(seq_lens: Sequence[int], num_splits: int, tile: int = 512) -> np.ndarray:
    """Static split-KV map: min(num_splits, tiles) chunks per request, one worker each."""
    lens = _i32_host(seq_lens)
    return _plan_call(lib().attn_plan_static, "attn_plan_static", _ptr_i32(lens), len(lens), num_splits, tile)


def attn_plan_lpt(seq_lens: Sequence[int], num_workers: int, tile: int = 512) -> np.ndarray:
    """LPT comparison map (version 2, with a per-worker order list)."""
    lens = _i32_host(seq_lens)
    return _plan_call(lib().attn_plan_lpt, "attn_plan_lpt", _ptr_i32(lens), len(lens), num_workers, tile)


def attn_plan_weighted(seq_lens: Sequence[int], num_workers: int, tile: int = 512, split_cost: int = 0) -> np.ndarray:
    """Cost-weighted contiguous fill (version-1 map): tile cost = KV tokens, plus split_cost on each
    request's first tile; tile i to worker floor(W (2 P_i + c_i) / (2 C))."""
    lens = _i32_host(seq_lens)
    return _plan_call(lib().attn_plan_weighted, "attn_plan_weighted", _ptr_i32(lens), len(lens), num_workers, tile,
                      split_cost)


MAP_VERSION_PLACED = 3     # lbsa.h LBSA_MAP_VERSION_PLACED
RATE_MAX = 1 << 20         # lbsa.h LBSA_RATE_MAX


def attn_plan_rated(seq_lens: Sequence[int], num_workers: int, rates: Sequence[int], tile: int = 512,
                    split_cost: int = 0) -> np.ndarray:
    """Rate-proportional contiguous fill (version-3 map, list-major workgroup order): worker w's
    share of the cost line is proportional to rates[w] (ints in [0, RATE_MAX], not all zero)."""
    lens = _i32_host(seq_lens)
    r = _i32_host(rates)
    if len(r) != num_workers:
        raise ValueError(f"attn_plan_rated: need {num_workers} rates, got {len(r)}")
    return _plan_call(lib().attn_plan_rated, "attn_plan_rated", _ptr_i32(lens), len(lens), num_workers, tile,
                      split_cost, _ptr_i32(r))


def attn_plan_prefill(q_lens: Sequence[int], kv_lens: Sequence[int], num_workers: int, q_tile: int = 128,
                      kv_tile: int = 512, causal: bool = True) -> np.ndarray:
    ql, kl = _i32_host(q_lens), _i32_host(kv_lens)
    if len(ql) != len(kl):
        raise ValueError("q_lens and kv_lens differ in length")
    return _plan_call(lib().attn_plan_prefill, "attn_plan_prefill", _ptr_i32(ql), _ptr_i32(kl), len(ql),
                      num_workers, q_tile, kv_tile, int(bool(causal)))


def attn_plan_device(seq_lens: torch.Tensor, num_workers: int, tile: int, map_dev: torch.Tensor,
                     stream=None) -> None:
    """Build the attn_plan map on the device (asynchronous, on the stream) from device lengths
    seq_lens int32[B] into map_dev int32[capacity]; map_dev[0] reports data errors (see lbsa.h)."""
    _need(seq_lens, torch.int32, "seq_lens", map_dev.device)
    _need(map_dev, torch.int32, "map", map_dev.device)
    st = lib().attn_plan_device(_dptr(seq_lens), seq_lens.numel(), num_workers, tile, _dptr(map_dev), map_dev.numel(),
                                _stream(stream))
    _check(st, "attn_plan_device")


def device_map_words(num_units: int, num_workers: int) -> int:
    """Map words that always suffice for a device-built decode map (S <= W + U - 1)."""
    return attn_map_words(num_units, num_workers, 2**62)


def attn_query_workers(device: int = 0, head_groups: int = 8, kv_dtype: int = KV_BF16) -> int:
    out = _c_i32(0)
    _check(lib().attn_query_workers(device, head_groups, kv_dtype, ctypes.byref(out)), "attn_query_workers")
    return out.value


def _dptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str, dev=None) -> None:
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous {dtype} GPU tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name}: on {t.device}, expected {dev}")


def map_header(map_host: np.ndarray) -> dict:
    keys = ("version", "B", "W", "kv_tile", "S", "T", "q_tile", "U")
    return dict(zip(keys, (int(x) for x in map_host[:8])))


def max_splits_of(map_host: np.ndarray) -> int:
    """Largest number of partial slots of one unit in a host work map."""
    hdr = map_header(map_host)
    o = 8 + hdr["W"] + 1
    ptr = np.asarray(map_host[o:o + hdr["U"] + 1], dtype=np.int64)
    return int(np.max(np.diff(ptr))) if hdr["U"] > 0 else 0


def _cache_geometry(k_cache: torch.Tensor, v_cache: torch.Tensor, head_dim: int):
    """(num_pages, Hkv, page_size) of caches in the blocked layout (rows of 64 bytes, w elements):
    k_cache [P, Hkv, D/w, page, w], v_cache [P, Hkv, page/w, D, w]."""
    w = 64 // k_cache.element_size()
    if k_cache.dim() != 5 or v_cache.dim() != 5:
        raise ValueError("k_cache/v_cache: need the blocked layout [P, Hkv, D/w, page, w] / [P, Hkv, page/w, D, w]")
    P, Hkv, kt, page, wk = k_cache.shape
    if wk != w or kt * w != head_dim or page % w or tuple(v_cache.shape) != (P, Hkv, page // w, head_dim, w):
        raise ValueError(f"k_cache {tuple(k_cache.shape)} / v_cache {tuple(v_cache.shape)} do not match the blocked "
                         f"layout [P, Hkv, D/w, page, w] / [P, Hkv, page/w, D, w] with w = {w}, D = {head_dim}")
    return P, Hkv, page


def _check_partial_sizes(q, part_m, part_l, part_o, slots: int, rows_per_slot: int, what: str) -> None:
    """Every partial buffer holds slots x rows_per_slot rows of Hq heads (o: x D).  Checked before any
    device check, so an undersized buffer is refused whatever device it is on."""
    if q.dim() != 3:
        raise ValueError("q: need [rows, Hq, D]")
    Hq, D = q.shape[1], q.shape[2]
    n = slots * rows_per_slot * Hq
    for name, t, need in (("part_m", part_m, n), ("part_l", part_l, n), ("part_o", part_o, n * D)):
        if t.numel() < need:
            raise ValueError(f"{name}: {t.numel()} elements, smaller than {what} ({need})")


def _check_decode_args(q, k_cache, v_cache, block_table, seq_lens, map_dev, num_workers, num_segments, head_groups,
                       part_m, part_l, part_o, timing, cache_dtype):
    _check_partial_sizes(q, part_m, part_l, part_o, num_segments, 1, "num_segments")
    dev = q.device
    _need(q, torch.bfloat16, "q", dev)
    _need(k_cache, cache_dtype, "k_cache", dev)
    _need(v_cache, cache_dtype, "v_cache", dev)
    _need(block_table, torch.int32, "block_table", dev)
    _need(seq_lens, torch.int32, "seq_lens", dev)
    _need(map_dev, torch.int32, "map", dev)
    for name, t in (("part_m", part_m), ("part_l", part_l), ("part_o", part_o)):
        _need(t, torch.float32, name, dev)
    B, Hq, D = q.shape
    P, Hkv, page = _cache_geometry(k_cache, v_cache, D)
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("block_table/seq_lens do not match the batch")
    if timing is not None:
        _need(timing, torch.int64, "timing", dev)
        if timing.numel() < num_workers * head_groups * 4:
            raise ValueError("timing buffer too small")
    return B, Hq, D, P, Hkv, page


def attn_splitkv(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, map_dev: torch.Tensor, num_workers: int, num_segments: int,
                 head_groups: int, softmax_scale: float, part_m: torch.Tensor, part_l: torch.Tensor,
                 part_o: torch.Tensor, timing: Optional[torch.Tensor] = None, stream=None) -> None:
    """Launch the split-KV decode kernel.  Layouts: q [B, Hq, D]; k_cache [P, Hkv, D/32, page, 32] and
    v_cache [P, Hkv, page/32, D, 32] bf16 (blocked, see ``paged``); block_table [B, stride];
    part_m/l [S, Hq]; part_o [S, Hq, D]."""
    B, Hq, D, P, Hkv, page = _check_decode_args(q, k_cache, v_cache, block_table, seq_lens, map_dev, num_workers,
                                                num_segments, head_groups, part_m, part_l, part_o, timing,
                                                torch.bfloat16)
    st = lib().attn_splitkv(_dptr(q), _dptr(k_cache), _dptr(v_cache), _dptr(block_table), block_table.shape[1],
                            P, _dptr(seq_lens), _dptr(map_dev), num_workers, num_segments, head_groups, B, Hq,
                            Hkv, D, page, float(softmax_scale), _dptr(part_m), _dptr(part_l), _dptr(part_o),
                            _dptr(timing), _stream(stream))
    _check(st, "attn_splitkv")


def attn_splitkv_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                     v_scale: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, map_dev: torch.Tensor,
                     num_workers: int, num_segments: int, head_groups: int, softmax_scale: float,
                     part_m: torch.Tensor, part_l: torch.Tensor, part_o: torch.Tensor,
                     timing: Optional[torch.Tensor] = None, stream=None) -> None:
    """Launch the split-KV decode kernel over an 8-bit E4M3 cache: k_cache [P, Hkv, D/64, page, 64] and
    v_cache [P, Hkv, page/64, D, 64] uint8 codes (blocked, see ``paged``), k_scale/v_scale float32 [Hkv]
    (value = e4m3(code) * scale of the head)."""
    B, Hq, D, P, Hkv, page = _check_decode_args(q, k_cache, v_cache, block_table, seq_lens, map_dev, num_workers,
                                                num_segments, head_groups, part_m, part_l, part_o, timing,
                                                torch.uint8)
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t, torch.float32, name, q.device)
        if t.numel() != Hkv:
            raise ValueError(f"{name}: need one scale per KV head ({Hkv})")
    st = lib().attn_splitkv_fp8(_dptr(q), _dptr(k_cache), _dptr(v_cache), _dptr(k_scale), _dptr(v_scale),
                                _dptr(block_table), block_table.shape[1], P, _dptr(seq_lens), _dptr(map_dev),
                                num_workers, num_segments, head_groups, B, Hq, Hkv, D, page, float(softmax_scale),
                                _dptr(part_m), _dptr(part_l), _dptr(part_o), _dptr(timing), _stream(stream))
    _check(st, "attn_splitkv_fp8")


def attn_splitkv_claimed(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, map_dev: torch.Tensor, num_workers: int, num_segments: int,
                         resident_workgroups: int, claim_state: torch.Tensor, softmax_scale: float,
                         part_m: torch.Tensor, part_l: torch.Tensor, part_o: torch.Tensor, kv_scales=None,
                         timing: Optional[torch.Tensor] = None, stream=None) -> None:
    """Split-KV decode with run-time claiming: resident_workgroups one-wave workgroups take the map's
    (list, KV head) items from claim_state (device int32[2], zero before the first launch and left
    zero by every launch).  Same partials as attn_splitkv / attn_splitkv_fp8 over the same map."""
    fp8 = k_cache.dtype == torch.uint8
    B, Hq, D, P, Hkv, page = _check_decode_args(q, k_cache, v_cache, block_table, seq_lens, map_dev, num_workers,
                                                num_segments, 1, part_m, part_l, part_o, None,
                                                torch.uint8 if fp8 else torch.bfloat16)
    _need(claim_state, torch.int32, "claim_state", q.device)
    if claim_state.numel() < 2:
        raise ValueError("claim_state: need 2 int32")
    if timing is not None:
        _need(timing, torch.int64, "timing", q.device)
        if timing.numel() < resident_workgroups * 4:
            raise ValueError("timing buffer too small")
    ks = vs = None
    if fp8:
        if kv_scales is None:
            raise ValueError("an 8-bit cache needs kv_scales=(k_scale, v_scale)")
        ks, vs = kv_scales
        for name, t in (("k_scale", ks), ("v_scale", vs)):
            _need(t, torch.float32, name, q.device)
            if t.numel() != Hkv:
                raise ValueError(f"{name}: need one scale per KV head ({Hkv})")
    st = lib().attn_splitkv_claimed(_dptr(q), _dptr(k_cache), _dptr(v_cache), KV_FP8_E4M3 if fp8 else KV_BF16,
                                    _dptr(ks), _dptr(vs), _dptr(block_table), block_table.shape[1], P,
                                    _dptr(seq_lens), _dptr(map_dev), num_workers, num_segments, B, Hq, Hkv, D, page,
                                    float(softmax_scale), int(resident_workgroups), _dptr(claim_state),
                                    _dptr(part_m), _dptr(part_l), _dptr(part_o), _dptr(timing), _stream(stream))
    _check(st, "attn_splitkv_claimed")


def attn_splitkv_mtp(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                     q_lens: torch.Tensor, q_start: torch.Tensor, kv_lens: torch.Tensor, map_dev: torch.Tensor,
                     num_workers: int, num_segments: int, head_groups: int, rows_per_unit: int, softmax_scale: float,
                     part_m: torch.Tensor, part_l: torch.Tensor, part_o: torch.Tensor, kv_scales=None,
                     stream=None) -> None:
    """Multi-token decode: q [rows, Hq, D] with request b's q_lens[b] <= rows_per_unit rows from row
    q_start[b]; caches bf16, or uint8 E4M3 codes with kv_scales = (k_scale, v_scale); map from
    attn_plan_prefill(q_lens, kv_lens, W, q_tile=rows_per_unit); part_m/l [S, R, Hq], part_o [S, R, Hq, D]."""
    _check_partial_sizes(q, part_m, part_l, part_o, num_segments, int(rows_per_unit), "num_segments x rows_per_unit")
    fp8 = k_cache.dtype == torch.uint8
    dev = q.device
    _need(q, torch.bfloat16, "q", dev)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, torch.uint8 if fp8 else torch.bfloat16, name, dev)
    _need(block_table, torch.int32, "block_table", dev)
    for name, t in (("q_lens", q_lens), ("q_start", q_start), ("kv_lens", kv_lens), ("map", map_dev)):
        _need(t, torch.int32, name, dev)
    for name, t in (("part_m", part_m), ("part_l", part_l), ("part_o", part_o)):
        _need(t, torch.float32, name, dev)
    rows, Hq, D = q.shape
    P, Hkv, page = _cache_geometry(k_cache, v_cache, D)
    B = q_lens.numel()
    if block_table.dim() != 2 or block_table.shape[0] != B or q_start.numel() != B or kv_lens.numel() != B:
        raise ValueError("block_table/q_start/kv_lens do not match the batch")
    R = int(rows_per_unit)
    ks = vs = None
    if fp8:
        if kv_scales is None:
            raise ValueError("an 8-bit cache needs kv_scales=(k_scale, v_scale)")
        ks, vs = kv_scales
        for name, t in (("k_scale", ks), ("v_scale", vs)):
            _need(t, torch.float32, name, dev)
            if t.numel() != Hkv:
                raise ValueError(f"{name}: need one scale per KV head ({Hkv})")
    st = lib().attn_splitkv_mtp(_dptr(q), _dptr(k_cache), _dptr(v_cache), KV_FP8_E4M3 if fp8 else KV_BF16,
                                _dptr(ks), _dptr(vs), _dptr(block_table), block_table.shape[1], P, _dptr(q_lens),
                                _dptr(q_start), _dptr(kv_lens), _dptr(map_dev), num_workers, num_segments,
                                head_groups, B, Hq, Hkv, D, page, R, float(softmax_scale), _dptr(part_m),
                                _dptr(part_l), _dptr(part_o), _stream(stream))
    _check(st, "attn_splitkv_mtp")


def attn_splitkv_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                         q_lens: torch.Tensor, q_start: torch.Tensor, kv_lens: torch.Tensor, map_dev: torch.Tensor,
                         num_workers: int, num_segments: int, softmax_scale: float, part_m: torch.Tensor,
                         part_l: torch.Tensor, part_o: torch.Tensor, causal: bool = True, q_tile: int = 128,
                         exact_pv: Optional[bool] = None, stream=None) -> None:
    """Launch the chunked-prefill split-KV kernel.  q [rows, Hq, D]; caches as in attn_splitkv;
    q_lens/q_start/kv_lens [B]; part_m/l [S, q_tile, Hq]; part_o [S, q_tile, Hq, D].
    exact_pv: None (default) runs P.V in fp16 with every staged 64-key chunk of V checked, a chunk that
    fp16 does not hold exactly taking the bf16 path (V exact for every input); True runs every chunk
    on bf16 V with P as hi + lo bf16 parts; False takes the unchecked fp16 path, exact only for V = 0
    and 2^-17 <= |V| <= 65504."""
    _check_partial_sizes(q, part_m, part_l, part_o, num_segments, int(q_tile), "num_segments x q_tile")
    dev = q.device
    _need(q, torch.bfloat16, "q", dev)
    _need(k_cache, torch.bfloat16, "k_cache", dev)
    _need(v_cache, torch.bfloat16, "v_cache", dev)
    _need(block_table, torch.int32, "block_table", dev)
    for name, t in (("q_lens", q_lens), ("q_start", q_start), ("kv_lens", kv_lens), ("map", map_dev)):
        _need(t, torch.int32, name, dev)
    for name, t in (("part_m", part_m), ("part_l", part_l), ("part_o", part_o)):
        _need(t, torch.float32, name, dev)
    rows, Hq, D = q.shape
    P, Hkv, page = _cache_geometry(k_cache, v_cache, D)
    B = q_lens.numel()
    if block_table.dim() != 2 or block_table.shape[0] != B or q_start.numel() != B or kv_lens.numel() != B:
        raise ValueError("block_table/q_start/kv_lens do not match the batch")
    st = lib().attn_splitkv_prefill(_dptr(q), _dptr(k_cache), _dptr(v_cache), _dptr(block_table),
                                    block_table.shape[1], P, _dptr(q_lens), _dptr(q_start), _dptr(kv_lens),
                                    _dptr(map_dev), num_workers, num_segments, B, Hq, Hkv, D, page, q_tile,
                                    int(bool(causal)), float(softmax_scale), _dptr(part_m), _dptr(part_l),
                                    _dptr(part_o),
                                    0 if exact_pv is None else (PREFILL_EXACT_PV if exact_pv else PREFILL_F16_PV),
                                    _stream(stream))
    _check(st, "attn_splitkv_prefill")


def attn_store_kv(q_in: torch.Tensor, k_in: torch.Tensor, v_in: torch.Tensor, positions: torch.Tensor,
                  q_out: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                  q_norm_w: Optional[torch.Tensor] = None, k_norm_w: Optional[torch.Tensor] = None,
                  eps: float = 1e-6, rope_theta: float = 0.0, hadamard: bool = False, kv_scales=None,
                  stream=None) -> None:
    """Producer step: RMSNorm / RoPE / Hadamard on the new q and k, q to q_out (bf16), k and v stored
    at positions[b] of each request's pages (bf16 cache, or uint8 E4M3 with kv_scales)."""
    dev = q_in.device
    for name, t in (("q_in", q_in), ("k_in", k_in), ("v_in", v_in), ("q_out", q_out)):
        _need(t, torch.bfloat16, name, dev)
    fp8 = k_cache.dtype == torch.uint8
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, torch.uint8 if fp8 else torch.bfloat16, name, dev)
    _need(positions, torch.int32, "positions", dev)
    _need(block_table, torch.int32, "block_table", dev)
    B, Hq, D = q_in.shape
    P, Hkv, page = _cache_geometry(k_cache, v_cache, D)
    if tuple(k_in.shape) != (B, Hkv, D) or tuple(v_in.shape) != (B, Hkv, D) or tuple(q_out.shape) != (B, Hq, D):
        raise ValueError("q_in/k_in/v_in/q_out shapes do not match [B, Hq, D] / [B, Hkv, D]")
    if positions.numel() != B or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("positions/block_table do not match the batch")
    for name, t in (("q_norm_w", q_norm_w), ("k_norm_w", k_norm_w)):
        if t is not None:
            _need(t, torch.float32, name, dev)
            if t.numel() != D:
                raise ValueError(f"{name}: need {D} gains")
    ks = vs = None
    if fp8:
        if kv_scales is None:
            raise ValueError("an 8-bit cache needs kv_scales=(k_scale, v_scale)")
        ks, vs = kv_scales
        for name, t in (("k_scale", ks), ("v_scale", vs)):
            _need(t, torch.float32, name, dev)
            if t.numel() != Hkv:
                raise ValueError(f"{name}: need {Hkv} scales (one per KV head)")
    st = lib().attn_store_kv(_dptr(q_in), _dptr(k_in), _dptr(v_in), _dptr(q_norm_w), _dptr(k_norm_w), float(eps),
                             _dptr(positions), float(rope_theta), 1 if hadamard else 0, _dptr(q_out), _dptr(k_cache),
                             _dptr(v_cache), KV_FP8_E4M3 if fp8 else KV_BF16, _dptr(ks), _dptr(vs),
                             _dptr(block_table), block_table.shape[1], P, B, Hq, Hkv, D, page, _stream(stream))
    _check(st, "attn_store_kv")


def attn_store_kv_chunk(q_in: torch.Tensor, k_in: torch.Tensor, v_in: torch.Tensor, q_lens: torch.Tensor,
                        q_start: torch.Tensor, positions: torch.Tensor, max_q_len: int, q_out: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                        q_norm_w: Optional[torch.Tensor] = None, k_norm_w: Optional[torch.Tensor] = None,
                        eps: float = 1e-6, rope_theta: float = 0.0, hadamard: bool = False, kv_scales=None,
                        stream=None) -> None:
    """Producer step of a prefill chunk: request b's q_lens[b] new rows (from row q_start[b]) at
    positions positions[b] + j; q and k as attn_store_kv, V written in whole 64-byte cache rows."""
    dev = q_in.device
    for name, t in (("q_in", q_in), ("k_in", k_in), ("v_in", v_in), ("q_out", q_out)):
        _need(t, torch.bfloat16, name, dev)
    fp8 = k_cache.dtype == torch.uint8
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, torch.uint8 if fp8 else torch.bfloat16, name, dev)
    for name, t in (("q_lens", q_lens), ("q_start", q_start), ("positions", positions), ("block_table", block_table)):
        _need(t, torch.int32, name, dev)
    rows, Hq, D = q_in.shape
    P, Hkv, page = _cache_geometry(k_cache, v_cache, D)
    B = q_lens.numel()
    if tuple(k_in.shape) != (rows, Hkv, D) or tuple(v_in.shape) != (rows, Hkv, D) or tuple(q_out.shape) != (rows, Hq, D):
        raise ValueError("q_in/k_in/v_in/q_out shapes do not match [rows, Hq, D] / [rows, Hkv, D]")
    if q_start.numel() != B or positions.numel() != B or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("q_start/positions/block_table do not match the batch")
    for name, t in (("q_norm_w", q_norm_w), ("k_norm_w", k_norm_w)):
        if t is not None:
            _need(t, torch.float32, name, dev)
            if t.numel() != D:
                raise ValueError(f"{name}: need {D} gains")
    ks = vs = None
    if fp8:
        if kv_scales is None:
            raise ValueError("an 8-bit cache needs kv_scales=(k_scale, v_scale)")
        ks, vs = kv_scales
        for name, t in (("k_scale", ks), ("v_scale", vs)):
            _need(t, torch.float32, name, dev)
            if t.numel() != Hkv:
                raise ValueError(f"{name}: need {Hkv} scales (one per KV head)")
    st = lib().attn_store_kv_chunk(_dptr(q_in), _dptr(k_in), _dptr(v_in), _dptr(q_norm_w), _dptr(k_norm_w),
                                   float(eps), _dptr(q_lens), _dptr(q_start), _dptr(positions), int(max_q_len),
                                   float(rope_theta), 1 if hadamard else 0, _dptr(q_out), _dptr(k_cache),
                                   _dptr(v_cache), KV_FP8_E4M3 if fp8 else KV_BF16, _dptr(ks), _dptr(vs),
                                   _dptr(block_table), block_table.shape[1], P, B, Hq, Hkv, D, page, _stream(stream))
    _check(st, "attn_store_kv_chunk")


def attn_kv_layout(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor, dst_v: torch.Tensor,
                   to_blocked: bool = True, stream=None) -> None:
    """Convert a paged KV cache between the token-major layout [P, Hkv, page, D] and the blocked layout
    the attention kernels read ([P, Hkv, D/w, page, w] and [P, Hkv, page/w, D, w]); to_blocked=False
    converts back.  bf16 or uint8 (E4M3 codes); out of place."""
    tm, bl = (src_k, dst_k) if to_blocked else (dst_k, src_k)
    dev = src_k.device
    dtype = src_k.dtype
    for name, t in (("src_k", src_k), ("src_v", src_v), ("dst_k", dst_k), ("dst_v", dst_v)):
        _need(t, dtype, name, dev)
    if dtype not in (torch.bfloat16, torch.uint8) or tm.dim() != 4:
        raise ValueError("token-major caches: bf16 or uint8 [P, Hkv, page, D]")
    P, Hkv, page, D = tm.shape
    want_k = (P, Hkv, D // (64 // tm.element_size()), page, 64 // tm.element_size())
    want_v = (P, Hkv, page // (64 // tm.element_size()), D, 64 // tm.element_size())
    bl_v = dst_v if to_blocked else src_v
    tm_v = src_v if to_blocked else dst_v
    if tuple(bl.shape) != want_k or tuple(bl_v.shape) != want_v or tuple(tm_v.shape) != tuple(tm.shape):
        raise ValueError(f"blocked caches must be {want_k} / {want_v} for a token-major {tuple(tm.shape)}")
    st = lib().attn_kv_layout(_dptr(src_k), _dptr(src_v), _dptr(dst_k), _dptr(dst_v), P, Hkv, page, D,
                              KV_FP8_E4M3 if dtype == torch.uint8 else KV_BF16, 0 if to_blocked else 1,
                              _stream(stream))
    _check(st, "attn_kv_layout")


def attn_combine(part_m: torch.Tensor, part_l: torch.Tensor, part_o: torch.Tensor, map_dev: torch.Tensor,
                 num_units: int, out: torch.Tensor, rows_per_unit: int = 1, q_lens: Optional[torch.Tensor] = None,
                 q_start: Optional[torch.Tensor] = None, max_splits: int = 0, stream=None) -> None:
    """Merge partials into out [rows, Hq, D] (fp32 or bf16).  max_splits: largest slot count of a unit
    (a launch-shape hint; see max_splits_of)."""
    dev = out.device
    for name, t in (("part_m", part_m), ("part_l", part_l), ("part_o", part_o)):
        _need(t, torch.float32, name, dev)
    _need(map_dev, torch.int32, "map", dev)
    if out.dtype not in (torch.float32, torch.bfloat16) or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out: need a contiguous fp32 or bf16 GPU tensor")
    if q_lens is not None:
        _need(q_lens, torch.int32, "q_lens", dev)
        _need(q_start, torch.int32, "q_start", dev)
    Hq, D = out.shape[-2], out.shape[-1]
    st = lib().attn_combine(_dptr(part_m), _dptr(part_l), _dptr(part_o), _dptr(map_dev), num_units, rows_per_unit,
                            _dptr(q_lens), _dptr(q_start), Hq, D, _dptr(out),
                            1 if out.dtype == torch.bfloat16 else 0, int(max_splits), _stream(stream))
    _check(st, "attn_combine")


def attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                        seq_lens: torch.Tensor, map_dev: torch.Tensor, num_workers: int, num_segments: int,
                        head_groups: int, softmax_scale: float, out: torch.Tensor, max_splits: int = 0,
                        kv_scales=None, stream=None) -> None:
    """Split-KV decode plus combine with the partials in the library's own fixed device array (no
    allocation anywhere, this binding included): for callers that cannot allocate.  Caches bf16, or
    uint8 E4M3 codes with kv_scales = (k_scale, v_scale); out fp32 or bf16 [B, Hq, D].  Calls that
    may overlap on one GPU race (they share its array)."""
    fp8 = k_cache.dtype == torch.uint8
    dev = q.device
    _need(q, torch.bfloat16, "q", dev)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, torch.uint8 if fp8 else torch.bfloat16, name, dev)
    _need(block_table, torch.int32, "block_table", dev)
    _need(seq_lens, torch.int32, "seq_lens", dev)
    _need(map_dev, torch.int32, "map", dev)
    if out.dtype not in (torch.float32, torch.bfloat16) or not out.is_contiguous() or out.device != dev:
        raise ValueError("out: need a contiguous fp32 or bf16 tensor on q's device")
    B, Hq, D = q.shape
    P, Hkv, page = _cache_geometry(k_cache, v_cache, D)
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.numel() != B or tuple(out.shape) != (B, Hq, D):
        raise ValueError("block_table/seq_lens/out do not match the batch")
    ks = vs = None
    if fp8:
        if kv_scales is None:
            raise ValueError("an 8-bit cache needs kv_scales=(k_scale, v_scale)")
        ks, vs = kv_scales
        for name, t in (("k_scale", ks), ("v_scale", vs)):
            _need(t, torch.float32, name, dev)
            if t.numel() != Hkv:
                raise ValueError(f"{name}: need one scale per KV head ({Hkv})")
    st = lib().attn_decode_noalloc(_dptr(q), _dptr(k_cache), _dptr(v_cache), KV_FP8_E4M3 if fp8 else KV_BF16,
                                   _dptr(ks), _dptr(vs), _dptr(block_table), block_table.shape[1], P,
                                   _dptr(seq_lens), _dptr(map_dev), num_workers, num_segments, head_groups, B, Hq,
                                   Hkv, D, page, float(softmax_scale), int(max_splits), _dptr(out),
                                   1 if out.dtype == torch.bfloat16 else 0, _stream(stream))
    _check(st, "attn_decode_noalloc")


def attn_probe_stream_read(buf: torch.Tensor, blocks: int, sink: torch.Tensor, stream=None) -> None:
    """Read all of ``buf`` once (measurement helper: the device's streaming-read ceiling)."""
    if not buf.is_cuda or not buf.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < blocks * 256:
        raise ValueError("attn_probe_stream_read: need a contiguous GPU buffer and an int32 sink of blocks*256")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().attn_probe_stream_read(_dptr(buf), nbytes - nbytes % 16, blocks, _dptr(sink), _stream(stream)),
           "attn_probe_stream_read")


def attn_probe_stream_read_rated(buf: torch.Tensor, blocks: int, xcd_rates: Sequence[int], sink: torch.Tensor,
                                 stream=None) -> None:
    """Read all of ``buf`` once, XCD x's workgroups taking a share in proportion to xcd_rates[x]
    (measurement helper: the streaming-read ceiling when work follows the XCDs' rates)."""
    if not buf.is_cuda or not buf.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < blocks * 256:
        raise ValueError("attn_probe_stream_read_rated: need a contiguous GPU buffer and an int32 sink of blocks*256")
    r = _i32_host(xcd_rates)
    if len(r) != 8:
        raise ValueError("attn_probe_stream_read_rated: need eight rates, one per XCD")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().attn_probe_stream_read_rated(_dptr(buf), nbytes - nbytes % 16, blocks, _ptr_i32(r), _dptr(sink),
                                              _stream(stream)), "attn_probe_stream_read_rated")


def attn_probe_mfma_rate(iters: int, blocks: int, sink: torch.Tensor, stream=None) -> int:
    """Run the matrix-core rate probe (measurement helper); returns the flops of the launch."""
    if not sink.is_cuda or sink.dtype != torch.int32 or not sink.is_contiguous() or sink.numel() < blocks * 256:
        raise ValueError("attn_probe_mfma_rate: need a contiguous int32 GPU sink of blocks*256")
    _check(lib().attn_probe_mfma_rate(int(iters), int(blocks), _dptr(sink), _stream(stream)), "attn_probe_mfma_rate")
    return int(blocks) * 4 * int(iters) * 8 * 16384
