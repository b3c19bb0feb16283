"""Seeded synthetic inputs for load-balanced split-KV attention.

Shared by both sides of every parity check (the float64 oracle and the GPU
library's harness).  This module holds random draws and the workload recipes
only: it contains none of the method's arithmetic (no tile cut, no scheduling,
no softmax), and it imports neither the oracle nor the GPU library.

Shapes follow the model the pages describe ([P3] "Hy3 Preview AI Infra 推理优化
精读笔记" §2: 64 attention heads, 8 KV heads, head dim 128) and the request
length mix their workload section gives (§1 and §12.1 of the same page: inputs
up to about 192K tokens, buckets 1K/4K/16K/64K/128K mixed in one batch; [P3] §6
and [P1] §3.4: prefix-cache reuse, about 80% hit rate).  The pages measure on a
private production trace that is not available; these synthetic batches stand
in for it.

Every value is drawn N(0, 1) in float32 from a seeded ``torch.Generator`` on the
CPU and rounded to bfloat16 (round to nearest even); both sides then see the
same bf16 values.  Seeds: ``seed_for(workload_id, stream, index)`` with streams
0 = lengths / order, 1 = page permutation, 2 = Q, 3 = K, 4 = V, 5 = the per-head
scales of an 8-bit cache; K and V are drawn per request so a long batch can be
generated and checked one request at a time.  An 8-bit (E4M3) cache holds the
same K and V draws, quantised per KV head (``Workload.kv_fp8``).

Score profiles (``Workload.profile``) reshape the same draws into inputs whose softmax is peaked or
moves, so that the kernels' online softmax must move its running maximum part-way through a split
(the exact merge of split partials, [P3] §3.1 方案 step 5 and §14 "Split-KV"):

* ``q8`` / ``q16``: q multiplied by 8 or 16 (exact in bf16): scores with a spread of 8 or 16;
* ``ramp``: q's dim 0 set to 64 and K's dim 0 to 0.02 t at token t: scores climb by about 7.2
  per 64 tokens along every request;
* ``spike``: q's dim 0 set to 8 and, at tokens t = 650 (mod 700), K's dim 0 set to 15 + 8.5 j
  (the j-th such token): late dominant keys, each about 6 above the previous one;
* ``vsmall`` / ``vlarge``: V multiplied by 1e-6 or 1e5 before its bf16 rounding (value range);
  ``vlow`` / ``vhigh``: V times 2^-10 or 2^13 (small and large magnitudes that fp16 still holds).

An 8-bit cache of a profile with larger K or V takes its per-head scales times a power of two (or
the V factor) that keeps the values inside the E4M3 range.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

HQ = 64
HKV = 8
HEAD_DIM = 128
PAGE = 64
TILE = 512
Q_TILE = 128

STREAM_LENGTHS, STREAM_PAGES, STREAM_Q, STREAM_K, STREAM_V, STREAM_SCALES = 0, 1, 2, 3, 4, 5
E4M3_MAX = 448.0


def seed_for(workload_id: int, stream: int, index: int = 0) -> int:
    return int(workload_id * 1_000_000 + stream * 10_000 + index)


def randn_f32(shape, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def randn_bf16(shape, seed: int) -> torch.Tensor:
    return randn_f32(shape, seed).to(torch.bfloat16)


def to_e4m3_codes(x: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """Input recipe of an 8-bit cache (the producer's job, not the attention's): x / scale per KV
    head (dim 1), clamped to the E4M3 range and rounded to nearest even by torch's float8_e4m3fn
    conversion; returns the codes as uint8."""
    y = (x / scale[None, :, None]).clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


PROFILES = ("normal", "q8", "q16", "ramp", "spike", "vsmall", "vlarge", "vlow", "vhigh")
RAMP_Q, RAMP_SLOPE = 64.0, 0.02
SPIKE_Q, SPIKE_PERIOD, SPIKE_AT, SPIKE_K0, SPIKE_STEP = 8.0, 700, 650, 15.0, 8.5
V_FACTOR = {"vsmall": 1e-6, "vlarge": 1e5, "vlow": 2.0 ** -10, "vhigh": 2.0 ** 13}


@dataclass
class Workload:
    """One synthetic batch: KV lengths (and, for prefill, query-chunk lengths)."""
    name: str
    workload_id: int
    kv_lens: List[int]
    q_lens: List[int]                 # 1 per request for decode
    kind: str = "decode"              # "decode" (one query row), "prefill" or "mtp" (q_lens rows each)
    workers: Optional[int] = None     # fixed worker count (None: from the device)
    paged: bool = True                # False: identity block table (contiguous pages)
    hq: int = HQ
    hkv: int = HKV
    head_dim: int = HEAD_DIM
    meta: dict = field(default_factory=dict)
    profile: str = "normal"           # score profile (module docstring)

    @property
    def batch(self) -> int:
        return len(self.kv_lens)

    def q(self, b: Optional[int] = None) -> torch.Tensor:
        """Decode: all queries [B, Hq, D].  Prefill and multi-token decode: request b's rows
        [q_len_b, Hq, D]."""
        if self.kind == "decode":
            x = randn_f32((self.batch, self.hq, self.head_dim), seed_for(self.workload_id, STREAM_Q))
        else:
            x = randn_f32((self.q_lens[b], self.hq, self.head_dim), seed_for(self.workload_id, STREAM_Q, b))
        return self._shape_q(x).to(torch.bfloat16)

    def _shape_q(self, x: torch.Tensor) -> torch.Tensor:
        if self.profile == "q8":
            return x * 8
        if self.profile == "q16":
            return x * 16
        if self.profile in ("ramp", "spike"):
            x[..., 0] = RAMP_Q if self.profile == "ramp" else SPIKE_Q
        return x

    def _kv_f32(self, b: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """Request b's keys and values [L_b, Hkv, D] in float32, shaped by the profile."""
        L = self.kv_lens[b]
        k = randn_f32((L, self.hkv, self.head_dim), seed_for(self.workload_id, STREAM_K, b))
        v = randn_f32((L, self.hkv, self.head_dim), seed_for(self.workload_id, STREAM_V, b))
        if self.profile == "ramp":
            k[:, :, 0] = RAMP_SLOPE * torch.arange(L, dtype=torch.float32)[:, None]
        elif self.profile == "spike":
            at = torch.arange(SPIKE_AT, L, SPIKE_PERIOD)
            k[at, :, 0] = (SPIKE_K0 + SPIKE_STEP * torch.arange(len(at), dtype=torch.float32))[:, None]
        elif self.profile in V_FACTOR:
            v = v * V_FACTOR[self.profile]
        return k, v

    def kv(self, b: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """Request b's keys and values, each [L_b, Hkv, D] bf16, token-major."""
        k, v = self._kv_f32(b)
        return k.to(torch.bfloat16), v.to(torch.bfloat16)

    def _k_range(self) -> float:
        """Largest |K| the profile produces (over the batch), for the 8-bit cache's scales."""
        L = max(self.kv_lens) if self.kv_lens else 0
        if self.profile == "ramp":
            return RAMP_SLOPE * L
        if self.profile == "spike":
            return SPIKE_K0 + SPIKE_STEP * max(0, (L - SPIKE_AT + SPIKE_PERIOD - 1) // SPIKE_PERIOD)
        return 0.0

    def kv_scales(self) -> Tuple[torch.Tensor, torch.Tensor]:
        """Per-KV-head float32 scales of the 8-bit cache, K and V: 2^u with u ~ U[-6.5, -5.5], about
        what an amax / 448 calibration gives for N(0, 1) values, and different for every head; a
        profile with larger K takes them times the power of two that covers its largest K, one with
        scaled V times its V factor."""
        g = torch.Generator(device="cpu")
        g.manual_seed(seed_for(self.workload_id, STREAM_SCALES))
        u = torch.rand(2, self.hkv, generator=g, dtype=torch.float32) - 6.5
        s = torch.exp2(u)
        kr = self._k_range()
        if kr > 5.0:
            s[0] *= 2.0 ** math.ceil(math.log2(kr / 5.0))
        if self.profile in V_FACTOR:
            s[1] *= V_FACTOR[self.profile]
        return s[0].clone(), s[1].clone()

    def kv_fp8(self, b: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """Request b's keys and values as E4M3 codes [L_b, Hkv, D] uint8: the same draws as ``kv``
        (before their bf16 rounding), quantised with ``kv_scales``."""
        ks, vs = self.kv_scales()
        k, v = self._kv_f32(b)
        return to_e4m3_codes(k, ks), to_e4m3_codes(v, vs)

    def page_permutation(self, num_pages: int) -> torch.Tensor:
        """Physical page for each logical page (a seeded shuffle; identity when not paged)."""
        if not self.paged:
            return torch.arange(num_pages)
        g = torch.Generator(device="cpu")
        g.manual_seed(seed_for(self.workload_id, STREAM_PAGES))
        return torch.randperm(num_pages, generator=g)

    def kv_bytes(self) -> int:
        return sum(self.kv_lens) * self.hkv * self.head_dim * 2 * 2


def _shuffled(values: List[int], seed: int) -> List[int]:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    order = torch.randperm(len(values), generator=g).tolist()
    return [values[i] for i in order]


def tiny() -> Workload:
    """The pages' worked example ([P3] §3.1 方案): KV lengths 1024, 5120, 2048; 4 workers."""
    return Workload("tiny", 1, [1024, 5120, 2048], [1, 1, 1], workers=4, paged=False)


def uniform() -> Workload:
    """64 requests at 8192 tokens each."""
    return Workload("uniform", 2, [8192] * 64, [1] * 64)


def mixed() -> Workload:
    """8 requests at each of 1K, 4K, 16K, 64K and 128K tokens (K = 1024), order shuffled."""
    lens = [n * 1024 for n in (1, 4, 16, 64, 128) for _ in range(8)]
    lens = _shuffled(lens, seed_for(3, STREAM_LENGTHS))
    return Workload("mixed", 3, lens, [1] * len(lens))


def mixed_tp8() -> Workload:
    """One GPU's share of the mixed batch under 8-way KV-head sharding: the same lengths, 8 query
    heads over 1 KV head (its own seeds)."""
    lens = [n * 1024 for n in (1, 4, 16, 64, 128) for _ in range(8)]
    lens = _shuffled(lens, seed_for(3, STREAM_LENGTHS))
    return Workload("mixed_tp8", 7, lens, [1] * len(lens), hq=8, hkv=1)


def long_tail() -> Workload:
    """One 192K-token request followed by 15 requests of uniform length in [1024, 2048]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(4, STREAM_LENGTHS))
    tail = torch.randint(1024, 2049, (15,), generator=g).tolist()
    lens = [196608] + tail
    return Workload("long_tail", 4, lens, [1] * len(lens))


def control() -> Workload:
    """The mixed batch's token count spread evenly: 40 requests of 43,622 tokens (control for the
    length mix: same KV bytes, no imbalance to remove)."""
    return Workload("control", 6, [43622] * 40, [1] * 40)


def prefill(chunk: int = 2048, requests: int = 8) -> Workload:
    """Chunked causal prefill: per request a ``chunk``-row query chunk after a cached prefix whose
    length is log-uniform in [8K, 128K] tokens."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(5, STREAM_LENGTHS))
    u = torch.rand(requests, generator=g, dtype=torch.float64).tolist()
    lo, hi = math.log(8192), math.log(131072)
    prefixes = [int(round(math.exp(lo + x * (hi - lo)))) for x in u]
    kv = [p + chunk for p in prefixes]
    return Workload("prefill", 5, kv, [chunk] * requests, kind="prefill", meta={"prefix": prefixes})


def random_decode(seed: int, batch: int, max_len: int, min_len: int = 0, hq: int = HQ, hkv: int = HKV,
                  head_dim: int = HEAD_DIM, paged: bool = True) -> Workload:
    """Small seeded decode batches for parity tests (ragged lengths, empty requests allowed)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(100 + seed, STREAM_LENGTHS))
    lens = torch.randint(min_len, max_len + 1, (batch,), generator=g).tolist()
    return Workload(f"random_decode_{seed}", 100 + seed, lens, [1] * batch, hq=hq, hkv=hkv,
                    head_dim=head_dim, paged=paged)


def random_prefill(seed: int, batch: int, max_prefix: int, max_chunk: int, hq: int = HQ,
                   hkv: int = HKV) -> Workload:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(200 + seed, STREAM_LENGTHS))
    prefix = torch.randint(0, max_prefix + 1, (batch,), generator=g).tolist()
    chunk = torch.randint(1, max_chunk + 1, (batch,), generator=g).tolist()
    return Workload(f"random_prefill_{seed}", 200 + seed, [p + c for p, c in zip(prefix, chunk)], chunk,
                    kind="prefill", meta={"prefix": prefix}, hq=hq, hkv=hkv)


def mtp(q_len: int = 4, base: str = "mixed") -> Workload:
    """Multi-token decode over the KV lengths of a decode batch: every request verifies q_len drafted
    tokens (its last q_len positions), as in a multi-token-prediction step ([P3] §7)."""
    src = BY_NAME[base]()
    return Workload(f"mtp{q_len}_{base}", 300 + src.workload_id, list(src.kv_lens), [q_len] * src.batch, kind="mtp")


def random_mtp(seed: int, batch: int, max_len: int, max_q: int = 4, min_len: int = 4) -> Workload:
    """Small seeded multi-token decode batches: ragged KV lengths and 0..max_q query rows each."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(400 + seed, STREAM_LENGTHS))
    lens = torch.randint(min_len, max_len + 1, (batch,), generator=g).tolist()
    qs = torch.randint(0, max_q + 1, (batch,), generator=g).tolist()
    qs = [min(q, L) for q, L in zip(qs, lens)]
    return Workload(f"random_mtp_{seed}", 400 + seed, lens, qs, kind="mtp")


BY_NAME = {"tiny": tiny, "uniform": uniform, "mixed": mixed, "long_tail": long_tail, "control": control,
           "prefill": prefill, "mixed_tp8": mixed_tp8}
