"""Reference attention in float64 (oracle; test infrastructure only).

The method reaches exactly the plain result: splitting a request's KV range into
pieces, computing a partial softmax per piece and merging the pieces is an exact
re-association of one softmax sum ([P3] §14 glossary "Split-KV": the KV axis of
a long attention is divided among several CTAs whose partial results are then
merged; [P3] §3.1 方案 step 5: a combine kernel merges the split-KV partials).
So the output oracle is the definition itself, evaluated in float64:

    s_t = scale * <q, k_t>,   p_t = exp(s_t - max_t s_t),   out = sum_t p_t v_t / sum_t p_t

over the keys a query row may see.  Grouped-query attention with Hq query heads
and Hkv KV heads ([P3] §2: 64 attention heads, 8 KV heads, head dim 128): query
head h reads KV head h // (Hq // Hkv).

Readings (where the pages are silent):

* inputs are bf16 values widened exactly to float64 by the caller;
* decode: one query row per request at position L - 1, which sees all L keys;
  L = 0 gives an all-zero output;
* chunked prefill over a cached prefix: the q_len query rows are the last q_len
  positions of a kv_len-token context, row j sits at kv_len - q_len + j and sees
  keys [0, kv_len - q_len + j] (causal), or all kv_len keys (non-causal);
* a partial ("split") result is (m, l, o): m = max scaled score over the piece
  (natural-log units), l = sum exp(s - m), o = sum exp(s - m) v (not divided by
  l); a piece with no visible key gives (-inf, 0, 0);
* combine: M = max m_s; w_s = exp(m_s - M) (0 when m_s = -inf); out =
  sum w_s o_s / sum w_s l_s, and 0 when every piece is empty.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

Partial = Tuple[np.ndarray, np.ndarray, np.ndarray]  # m [R, Hq], l [R, Hq], o [R, Hq, D]

_ROW_BLOCK = 64   # rows per block when scores would not fit in memory at once


def _visible_upto(rows: int, first_row: int, q_len: int, kv_len: int, causal: bool) -> np.ndarray:
    """Exclusive upper key bound for rows first_row .. first_row+rows-1 of a q_len-row chunk."""
    if causal:
        return kv_len - q_len + first_row + np.arange(rows) + 1
    return np.full(rows, kv_len)


def ref_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                  causal: bool = True) -> np.ndarray:
    """Exact attention of one request.

    q: [R, Hq, D] query rows (the last R positions of the context), k, v: [L, Hkv, D].
    Returns out [R, Hq, D] float64.
    """
    m, l, o = ref_partial(q, k, v, scale, 0, k.shape[0], causal)
    out = np.zeros_like(o)
    nz = l > 0
    out[nz] = o[nz] / l[nz][:, None]
    return out


def ref_partial(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                kv_begin: int, kv_end: int, causal: bool = True,
                first_row: int = 0, q_len: int | None = None) -> Partial:
    """Partial softmax of query rows over keys [kv_begin, kv_end) (and the mask).

    q holds rows first_row .. first_row+R-1 of a request's q_len-row chunk (default: the whole
    chunk).  Returns m [R, Hq] (-inf where no key is visible), l [R, Hq], o [R, Hq, D]
    (unnormalised).
    """
    q = np.asarray(q, dtype=np.float64)
    R, Hq, D = q.shape
    L, Hkv, Dk = k.shape
    if Dk != D or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    if q_len is None:
        q_len = R
    if first_row < 0 or first_row + R > q_len:
        raise ValueError("rows outside the chunk")
    upto = _visible_upto(R, first_row, q_len, L, causal)
    m = np.full((R, Hq), -np.inf)
    l = np.zeros((R, Hq))
    o = np.zeros((R, Hq, D))
    a, e = max(0, kv_begin), min(L, kv_end)
    if e <= a:
        return m, l, o
    for g in range(Hkv):
        kg = np.asarray(k[a:e, g, :], dtype=np.float64)          # [n, D]
        vg = np.asarray(v[a:e, g, :], dtype=np.float64)          # [n, D]
        pos = np.arange(a, e)
        for r0 in range(0, R, _ROW_BLOCK):
            r1 = min(R, r0 + _ROW_BLOCK)
            qg = q[r0:r1, g * group:(g + 1) * group, :]          # [r, group, D]
            s = scale * (qg.reshape(-1, D) @ kg.T)               # [r*group, n]
            s = s.reshape(r1 - r0, group, e - a)
            visible = pos[None, :] < upto[r0:r1, None]           # [r, n]
            s = np.where(visible[:, None, :], s, -np.inf)
            mx = s.max(axis=2)                                   # [r, group]
            has = np.isfinite(mx)
            p = np.where(has[:, :, None], np.exp(s - np.where(has, mx, 0.0)[:, :, None]), 0.0)
            m[r0:r1, g * group:(g + 1) * group] = mx
            l[r0:r1, g * group:(g + 1) * group] = p.sum(axis=2)
            o[r0:r1, g * group:(g + 1) * group, :] = (p.reshape(-1, e - a) @ vg).reshape(r1 - r0, group, D)
    return m, l, o


def ref_combine(parts: Sequence[Partial]) -> np.ndarray:
    """Merge partial results of the same query rows (the combine step)."""
    if not parts:
        raise ValueError("nothing to combine")
    ms = np.stack([p[0] for p in parts])                          # [S, R, Hq]
    ls = np.stack([p[1] for p in parts])
    os_ = np.stack([p[2] for p in parts])                         # [S, R, Hq, D]
    M = ms.max(axis=0)
    has = np.isfinite(M)
    w = np.where(np.isfinite(ms), np.exp(ms - np.where(has, M, 0.0)[None]), 0.0)
    Lsum = (w * ls).sum(axis=0)
    num = (w[..., None] * os_).sum(axis=0)
    out = np.zeros_like(num)
    nz = Lsum > 0
    out[nz] = num[nz] / Lsum[nz][:, None]
    return out


def ref_decode(q: np.ndarray, ks: Sequence[np.ndarray], vs: Sequence[np.ndarray], scale: float) -> np.ndarray:
    """Decode attention for a batch: q [B, Hq, D], ks[b], vs[b]: [L_b, Hkv, D]. Returns [B, Hq, D]."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        out[b] = ref_attention(q[b:b + 1], ks[b], vs[b], scale, causal=True)[0]
    return out


def ref_split_partials(words: np.ndarray, q_rows: Sequence[np.ndarray], ks: Sequence[np.ndarray],
                       vs: Sequence[np.ndarray], scale: float, causal: bool = True) -> List[Partial]:
    """One partial per segment of a work map, in slot order.

    q_rows[b]: [q_len_b, Hq, D] (decode: q_len_b = 1).  A segment (b, i, a, e) covers query rows
    [i*q_tile, min(q_len_b, (i+1)*q_tile)) of request b and keys [a, e).
    """
    from .plan import parse_map
    mp = parse_map(words)
    parts = []
    for b, i, a, e in mp.segs:
        qb = q_rows[b]
        r0, r1 = i * mp.q_tile, min(qb.shape[0], (i + 1) * mp.q_tile)
        parts.append(ref_partial(qb[r0:r1], ks[b], vs[b], scale, int(a), int(e), causal,
                                 first_row=r0, q_len=qb.shape[0]))
    return parts


def ref_from_map(words: np.ndarray, q_rows: Sequence[np.ndarray], ks: Sequence[np.ndarray],
                 vs: Sequence[np.ndarray], scale: float, causal: bool = True) -> List[np.ndarray]:
    """Split by the map, then combine per unit; returns per-request outputs [q_len_b, Hq, D]."""
    from .plan import parse_map
    mp = parse_map(words)
    parts = ref_split_partials(words, q_rows, ks, vs, scale, causal)
    outs = [np.zeros(np.asarray(qb).shape) for qb in q_rows]
    for u in range(mp.U):
        b, i = (int(x) for x in mp.units[u])
        r0, r1 = i * mp.q_tile, min(q_rows[b].shape[0], (i + 1) * mp.q_tile)
        sl = range(int(mp.unit_ptr[u]), int(mp.unit_ptr[u + 1]))
        if len(sl) == 0:
            continue
        outs[b][r0:r1] = ref_combine([parts[s] for s in sl])
    return outs


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
