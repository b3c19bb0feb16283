"""Paged KV-cache layout used by the kernels (torch plumbing, no attention arithmetic).

A cache holds ``num_pages`` physical pages of ``page_size`` tokens.  Each (page, KV head) is one
contiguous block (16 KiB of bf16, or 8 KiB of 8-bit codes, for page_size 64 and head dim 128):

* ``k_cache[page, head]`` is [page_size, D], token-major;
* ``v_cache[page, head]`` is [D, page_size], dim-major (V transposed inside the page), so that the
  attention kernel reads runs of consecutive tokens of one dim, the operand order of the P.V
  contraction.

``block_table[b, p]`` is the physical page that holds tokens [p*page_size, (p+1)*page_size) of
request b.
"""

from __future__ import annotations

from typing import Callable, List, Sequence, Tuple

import torch


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
    if P == 0:
        return (torch.zeros((1, Hkv, page_size, D), dtype=dtype, device=device),
                torch.zeros((1, Hkv, D, page_size), dtype=dtype, device=device),
                torch.zeros((B, 1), dtype=torch.int32, device=device))
    perm = permutation(P).to(torch.int64)
    k_cache = torch.empty((P, Hkv, page_size, D), dtype=dtype, device=device)
    v_cache = torch.empty((P, Hkv, D, page_size), dtype=dtype, device=device)
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
        L = seq_lens[b]
        if k.dtype != dtype or v.dtype != dtype:
            raise ValueError(f"request {b}: cache dtype {dtype}, got {k.dtype}/{v.dtype}")
        kp = torch.full((n * page_size, Hkv, D), pad_value, dtype=dtype, device=device)
        vp = torch.full((n * page_size, Hkv, D), pad_value, dtype=dtype, device=device)
        kp[:L] = k.to(device)
        vp[:L] = v.to(device)
        kp = kp.view(n, page_size, Hkv, D).permute(0, 2, 1, 3)      # [n, Hkv, page, D]
        vp = vp.view(n, page_size, Hkv, D).permute(0, 2, 3, 1)      # [n, Hkv, D, page]
        idx = phys.to(device)
        k_cache.index_copy_(0, idx, kp.contiguous())
        v_cache.index_copy_(0, idx, vp.contiguous())
        first += n
    return k_cache, v_cache, table.to(device)


def unpack_request(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor, b: int,
                   length: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Inverse of pack_paged for one request: token-major (k, v) [L, Hkv, D] (for checks)."""
    page_size = k_cache.shape[2]
    n = pages_for(length, page_size)
    idx = block_table[b, :n].to(torch.int64)
    k = k_cache.index_select(0, idx).permute(0, 2, 1, 3).reshape(n * page_size, k_cache.shape[1], -1)
    v = v_cache.index_select(0, idx).permute(0, 3, 1, 2).reshape(n * page_size, v_cache.shape[1], -1)
    return k[:length], v[:length]


def as_list(x) -> List[int]:
    return [int(v) for v in x]
