"""8-bit KV cache: the value of a stored element (oracle; test infrastructure only).

The pages run their production decode with an 8-bit KV cache ([P3] "Hy3 Preview AI Infra 推理优化
精读笔记" §1 and the §14 glossary entry "W8A8C8": weights, activations and the cache in 8 bits, the
exact format left to the implementation; §2 compression table and §8: attention in FP8; [P4]
"腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级" §一: the operator library supports BF16 and
several FP8 formats).  The attention itself is unchanged: it is the plain softmax attention of
``oracle.attention`` over the dequantised keys and values.

Readings (the pages fix neither the format nor the scale granularity):

* the format is OCP FP8 E4M3 ("e4m3fn"): one sign bit, four exponent bits with bias 7, three
  mantissa bits; exponent field 0 holds the subnormals m * 2^-9; there are no infinities and the
  two codes with every exponent and mantissa bit set (0x7F, 0xFF) are NaN; the largest finite
  magnitude is 448;
* one float32 scale per KV head for K and one for V, shared by every token and page of that head;
  the real value of a stored element of head g is ``e4m3(code) * scale[g]``.
"""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np

from .attention import ref_attention

E4M3_BIAS = 7
E4M3_MANT_BITS = 3


def e4m3_value(code: int) -> float:
    """The real number an E4M3 code stands for, from its bit fields."""
    if not 0 <= code <= 255:
        raise ValueError("an E4M3 code is one byte")
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> E4M3_MANT_BITS) & 0xF
    mant = code & 0x7
    if exp == 0xF and mant == 0x7:
        return math.nan
    if exp == 0:
        return sign * mant * 2.0 ** (1 - E4M3_BIAS - E4M3_MANT_BITS)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp - E4M3_BIAS)


def e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 codes."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_table()


def e4m3_to_float64(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise ValueError("codes must be uint8")
    return _TABLE[codes]


def dequantize_kv(codes: np.ndarray, scale: Sequence[float]) -> np.ndarray:
    """codes [L, Hkv, D] uint8, scale [Hkv] -> float64 [L, Hkv, D] = e4m3(code) * scale[head]."""
    vals = e4m3_to_float64(codes)
    scale = np.asarray(scale, dtype=np.float64)
    if vals.ndim != 3 or scale.shape != (vals.shape[1],):
        raise ValueError("codes must be [L, Hkv, D] with one scale per KV head")
    return vals * scale[None, :, None]


def ref_decode_fp8(q: np.ndarray, k_codes: Sequence[np.ndarray], v_codes: Sequence[np.ndarray],
                   k_scale: Sequence[float], v_scale: Sequence[float], scale: float) -> np.ndarray:
    """Decode attention over an FP8 cache: q [B, Hq, D] (bf16 values widened), codes [L_b, Hkv, D]."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        k = dequantize_kv(k_codes[b], k_scale)
        v = dequantize_kv(v_codes[b], v_scale)
        out[b] = ref_attention(q[b:b + 1], k, v, scale, causal=True)[0]
    return out
