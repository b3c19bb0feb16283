"""Paged KV-cache layout used by the kernels (torch plumbing, no attention arithmetic).

A cache holds ``num_pages`` physical pages of ``page_size`` tokens.  Each (page, KV head) is one
contiguous block (16 KiB of bf16, or 8 KiB of 8-bit codes, for page_size 64 and head dim 128),
stored in rows of 64 bytes (w = 64 / element bytes elements per row: 32 for bf16, 64 for 8-bit):

* ``k_cache[page, head]`` is [D / w, page_size, w]: dim tile, token, dim within the tile;
* ``v_cache[page, head]`` is [page_size / w, D, w]: token tile, dim, token within the tile.

So K is token-major inside each 64-byte dim tile and V is dim-major ("V transposed") inside each
64-byte token tile.  The attention kernels read 16-byte pieces that are MFMA operands; with this
blocking every load instruction covers whole 128-byte lines.

``block_table[b, p]`` is the physical page that holds tokens [p*page_size, (p+1)*page_size) of
request b.
"""

from __future__ import annotations

from typing import Callable, List, Sequence, Tuple

import torch

ROW_BYTES = 64


def row_elems(dtype: torch.dtype) -> int:
    return ROW_BYTES // torch.empty((), dtype=dtype).element_size()


def cache_shapes(num_pages: int, num_kv_heads: int, page_size: int, head_dim: int, dtype: torch.dtype):
    """Shapes of (k_cache, v_cache) in the blocked layout."""
    w = row_elems(dtype)
    if head_dim % w or page_size % w:
        raise ValueError(f"head_dim and page_size must be multiples of {w} for {dtype}")
    return ((num_pages, num_kv_heads, head_dim // w, page_size, w),
            (num_pages, num_kv_heads, page_size // w, head_dim, w))


def to_blocked(k: torch.Tensor, v: torch.Tensor, page_size: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Token-major k, v [n * page_size, Hkv, D] -> blocks [n, Hkv, D/w, page, w] and [n, Hkv, page/w, D, w]."""
    T, Hkv, D = k.shape
    n = T // page_size
    w = row_elems(k.dtype)
    kb = k.view(n, page_size, Hkv, D // w, w).permute(0, 2, 3, 1, 4)
    vb = v.view(n, page_size // w, w, Hkv, D).permute(0, 3, 1, 4, 2)
    return kb.contiguous(), vb.contiguous()


def from_blocked(kb: torch.Tensor, vb: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Inverse of to_blocked: token-major k, v [n * page_size, Hkv, D]."""
    n, Hkv, kt, page, w = kb.shape
    D = kt * w
    k = kb.permute(0, 3, 1, 2, 4).reshape(n * page, Hkv, D)
    v = vb.permute(0, 2, 4, 1, 3).reshape(n * page, Hkv, D)
    return k, v


def pages_for(length: int, page_size: int) -> int:
    return -(-length // page_size) if length > 0 else 0


def pack_paged(kv_of: Callable[[int], Tuple[torch.Tensor, torch.Tensor]], seq_lens: Sequence[int],
               page_size: int, num_kv_heads: int, head_dim: int, permutation: Callable[[int], torch.Tensor],
               device, pad_value: float = 0.0, dtype: torch.dtype = torch.bfloat16
               ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Build (k_cache, v_cache, block_table) on ``device``.

    kv_of(b) returns request b's (k, v), each [L_b, Hkv, D] of ``dtype`` (token-major): bf16, or
    uint8 E4M3 codes for an 8-bit cache.  permutation(P) returns the physical page of each of the P
    logical pages (batch order).  Tokens past a request's end inside its last page are filled with
    ``pad_value`` (a code for an 8-bit cache).
    """
    B = len(seq_lens)
    npages = [pages_for(L, page_size) for L in seq_lens]
    P = sum(npages)
    Hkv, D = num_kv_heads, head_dim
    kshape, vshape = cache_shapes(max(P, 1), Hkv, page_size, D, dtype)
    if P == 0:
        return (torch.zeros(kshape, dtype=dtype, device=device), torch.zeros(vshape, dtype=dtype, device=device),
                torch.zeros((B, 1), dtype=torch.int32, device=device))
    perm = permutation(P).to(torch.int64)
    k_cache = torch.empty(kshape, dtype=dtype, device=device)
    v_cache = torch.empty(vshape, dtype=dtype, device=device)
    stride = max(1, max(npages))
    table = torch.zeros((B, stride), dtype=torch.int32)
    first = 0
    for b in range(B):
        n = npages[b]
        if n == 0:
            continue
        phys = perm[first:first + n]
        table[b, :n] = phys.to(torch.int32)
        k, v = kv_of(b)
        if k.dtype != dtype or v.dtype != dtype:
            raise ValueError(f"request {b}: cache dtype {dtype}, got {k.dtype}/{v.dtype}")
        L = seq_lens[b]
        kp = torch.full((n * page_size, Hkv, D), pad_value, dtype=dtype, device=device)
        vp = torch.full((n * page_size, Hkv, D), pad_value, dtype=dtype, device=device)
        kp[:L] = k.to(device)
        vp[:L] = v.to(device)
        kb, vb = to_blocked(kp, vp, page_size)
        idx = phys.to(device)
        k_cache.index_copy_(0, idx, kb)
        v_cache.index_copy_(0, idx, vb)
        first += n
    return k_cache, v_cache, table.to(device)


def unpack_request(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor, b: int,
                   length: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Inverse of pack_paged for one request: token-major (k, v) [L, Hkv, D] (for checks)."""
    page_size = k_cache.shape[3]
    n = pages_for(length, page_size)
    idx = block_table[b, :n].to(torch.int64)
    k, v = from_blocked(k_cache.index_select(0, idx), v_cache.index_select(0, idx))
    return k[:length], v[:length]


def as_list(x) -> List[int]:
    return [int(v) for v in x]
