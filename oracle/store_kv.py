"""The producer step: normalise, rotate, quantise and store a step's new K/V (oracle; test
infrastructure only).

[P3] "Hy3 Preview AI Infra 推理优化精读笔记" §4.1 fuses the element-wise chain that follows the QKV
projection — RoPE, RMSNorm, Hadamard, quantisation and the KV-cache write — into one kernel, so
intermediates stay in registers and the cache is written directly in its low-bit format; §8 adds
that the query/key are Hadamard-rotated before quantisation to spread outliers.  The pages list the
steps but not their order or formulas.  Readings:

* per head vector x of length D (D even):
  1. RMSNorm (optional):  x <- x / sqrt(mean(x^2) + eps) * w,  w a per-dim gain shared by all heads
     of the same kind (one gain vector for q, one for k);
  2. RoPE (optional) at the token's position p, rotate-half pairing: for i < D/2, with
     a = p * theta^(-2i/D), (x_i, x_{i+D/2}) <- (x_i cos a - x_{i+D/2} sin a,
     x_{i+D/2} cos a + x_i sin a);
  3. Hadamard (optional): x <- H x / sqrt(D), H the Sylvester-ordered Walsh-Hadamard matrix
     (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]); applied to q and k alike, it leaves every q.k
     unchanged (H / sqrt(D) is orthogonal);
* q gets steps 1-3 and is returned in bf16 (round to nearest even); k gets steps 1-3 and v none; k
  and v are stored at the token's position of its request's paged cache, in bf16 or as E4M3 codes
  code = e4m3(clamp(x / scale[head], -448, 448)) rounded to nearest even (the format of
  ``oracle.fp8``).

Everything is computed in float64 and rounded once at the end.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .fp8 import e4m3_table


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x [..., D] -> x / sqrt(mean(x^2) + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, dtype=np.float64)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE.  x [N, H, D], pos [N]: pairs (i, i + D/2) rotated by pos * theta^(-2i/D)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    freq = theta ** (-2.0 * i / D)                                   # [D/2]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * freq[None, :]   # [N, D/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester-ordered Walsh-Hadamard matrix of order n (a power of two), entries +-1."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard(x: np.ndarray) -> np.ndarray:
    """x [..., D] -> (H x) / sqrt(D) along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    return x @ hadamard_matrix(D).T / math.sqrt(D)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even), as float64: x = m 2^e with
    0.5 <= |m| < 1 keeps round(m 2^8) 2^(e-8); below the normal range the step stays 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    step_exp = np.maximum(e - 8, -133)
    return np.round(np.ldexp(x, -step_exp)) * np.ldexp(1.0, step_exp)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """E4M3 code (uint8) of the finite value nearest to x, ties to the even code, |x| > 448 -> +-448,
    the sign bit kept (a negative value that rounds to zero gives 0x80).

    Written from the format's value table: the candidates are the 126 positive finite values and
    their negatives; the nearest wins and a tie goes to the code with an even mantissa."""
    table = e4m3_table()
    pos_codes = np.arange(0x00, 0x7F)               # 0x00 .. 0x7E: 0 .. 448, increasing
    pos_vals = table[pos_codes]
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    j = np.searchsorted(pos_vals, a)                # first value >= a
    j = np.clip(j, 1, len(pos_vals) - 1)
    lo, hi = pos_vals[j - 1], pos_vals[j]
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & ((pos_codes[j] & 1) == 0))
    code = np.where(pick_hi, pos_codes[j], pos_codes[j - 1])
    code = np.where(a == 0.0, 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)   # the sign is kept, -0 -> 0x80


def ref_store_kv(q: np.ndarray, k: np.ndarray, v: np.ndarray, positions: np.ndarray,
                 q_norm_w: Optional[np.ndarray], k_norm_w: Optional[np.ndarray], eps: float,
                 theta: float, use_hadamard: bool, k_scale: Optional[np.ndarray] = None,
                 v_scale: Optional[np.ndarray] = None):
    """One step's new tokens.  q [N, Hq, D], k and v [N, Hkv, D] (values of the projection output),
    positions [N].  Returns (q_out as bf16 values, k_store, v_store): the stored values are bf16
    values (float64 arrays) when no scales are given, else uint8 E4M3 codes."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q_norm_w is not None:
        q = rms_norm(q, q_norm_w, eps)
    if k_norm_w is not None:
        k = rms_norm(k, k_norm_w, eps)
    if theta > 0:
        q = rope(q, positions, theta)
        k = rope(k, positions, theta)
    if use_hadamard:
        q = hadamard(q)
        k = hadamard(k)
    q_out = round_bf16(q)
    if k_scale is None:
        return q_out, round_bf16(k), round_bf16(v)
    ks = np.asarray(k_scale, dtype=np.float64)[None, :, None]
    vs = np.asarray(v_scale, dtype=np.float64)[None, :, None]
    return q_out, e4m3_round(k / ks), e4m3_round(v / vs)
