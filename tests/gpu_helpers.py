"""Shared helpers for the GPU parity tests: seeded inputs in the kernels' layout, the fp64 oracle on
the same bf16 values, and the tolerance checks."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import workloads as WL
from load_balanced_split_attn_amd.paged import pack_paged
from oracle.attention import ref_attention

MAX_ABS = 1e-2
REL_RMS = 2e-3
SCALE = 1.0 / math.sqrt(128)


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def decode_inputs(wl: WL.Workload, device="cuda", page=64, pad_value=0.0):
    q = wl.q().to(device)
    k_cache, v_cache, bt = pack_paged(wl.kv, wl.kv_lens, page, wl.hkv, wl.head_dim, wl.page_permutation,
                                      device, pad_value=pad_value)
    return q, k_cache, v_cache, bt


def oracle_decode(wl: WL.Workload, requests=None, scale=SCALE):
    q = wl.q().to(torch.float64).numpy()
    out = {}
    for b in (range(wl.batch) if requests is None else requests):
        k, v = wl.kv(b)
        out[b] = ref_attention(q[b:b + 1], k.to(torch.float64).numpy(), v.to(torch.float64).numpy(), scale)[0]
    return out


def errors(got: np.ndarray, ref: np.ndarray):
    diff = got.astype(np.float64) - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS, rel_rms=REL_RMS):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ma, rr = errors(got, ref)
    assert ma <= max_abs and rr <= rel_rms, f"{what}: max_abs={ma:.3e} rel_rms={rr:.3e}"
    return ma, rr


def prefill_inputs(wl: WL.Workload, device="cuda", page=64, pad_value=0.0):
    q = torch.cat([wl.q(b) for b in range(wl.batch)], dim=0).to(device)
    k_cache, v_cache, bt = pack_paged(wl.kv, wl.kv_lens, page, wl.hkv, wl.head_dim, wl.page_permutation,
                                      device, pad_value=pad_value)
    return q, k_cache, v_cache, bt


def q_starts(wl: WL.Workload):
    starts, acc = [], 0
    for n in wl.q_lens:
        starts.append(acc)
        acc += n
    return starts


def oracle_prefill_rows(wl: WL.Workload, b: int, rows, causal=True, scale=SCALE):
    """fp64 oracle for selected rows of request b's chunk: {row: [Hq, D]}."""
    from oracle.attention import ref_partial
    q = wl.q(b).to(torch.float64).numpy()
    k, v = wl.kv(b)
    kd, vd = k.to(torch.float64).numpy(), v.to(torch.float64).numpy()
    out = {}
    for j in rows:
        m, l, o = ref_partial(q[j:j + 1], kd, vd, scale, 0, kd.shape[0], causal, first_row=j, q_len=q.shape[0])
        out[j] = o[0] / l[0][:, None]
    return out


def decode_inputs_fp8(wl: WL.Workload, device="cuda", page=64, pad_code=0):
    """q (bf16), the 8-bit caches (uint8 E4M3 codes, paged), block table and per-head scales."""
    q = wl.q().to(device)
    k_cache, v_cache, bt = pack_paged(wl.kv_fp8, wl.kv_lens, page, wl.hkv, wl.head_dim, wl.page_permutation,
                                      device, pad_value=pad_code, dtype=torch.uint8)
    ks, vs = wl.kv_scales()
    return q, k_cache, v_cache, bt, ks.to(device), vs.to(device)


def oracle_decode_fp8(wl: WL.Workload, requests=None, scale=SCALE):
    from oracle.fp8 import ref_decode_fp8
    q = wl.q().to(torch.float64).numpy()
    ks, vs = (s.to(torch.float64).numpy() for s in wl.kv_scales())
    out = {}
    for b in (range(wl.batch) if requests is None else requests):
        k, v = wl.kv_fp8(b)
        out[b] = ref_decode_fp8(q[b:b + 1], [k.numpy()], [v.numpy()], ks, vs, scale)[0]
    return out


def mtp_inputs(wl: WL.Workload, device="cuda", page=64, fp8=False, pad=0.0):
    """Rows of every request concatenated (q_start order), the paged caches and the block table
    (plus per-head scales for an 8-bit cache)."""
    rows = [wl.q(b) for b in range(wl.batch)]
    q = torch.cat(rows, dim=0).to(device) if sum(wl.q_lens) else torch.zeros((1, wl.hq, wl.head_dim),
                                                                                dtype=torch.bfloat16, device=device)
    if fp8:
        kc, vc, bt = pack_paged(wl.kv_fp8, wl.kv_lens, page, wl.hkv, wl.head_dim, wl.page_permutation, device,
                                pad_value=pad, dtype=torch.uint8)
        ks, vs = wl.kv_scales()
        return q, kc, vc, bt, (ks.to(device), vs.to(device))
    kc, vc, bt = pack_paged(wl.kv, wl.kv_lens, page, wl.hkv, wl.head_dim, wl.page_permutation, device,
                            pad_value=pad)
    return q, kc, vc, bt, None


def oracle_mtp(wl: WL.Workload, requests=None, fp8=False, scale=SCALE):
    """fp64 oracle: request b's q_len rows as the last positions of its context, causal.  {b: [q_len, Hq, D]}"""
    from oracle.fp8 import dequantize_kv
    out = {}
    if fp8:
        ks, vs = (s.to(torch.float64).numpy() for s in wl.kv_scales())
    for b in (range(wl.batch) if requests is None else requests):
        if wl.q_lens[b] == 0:
            continue
        q = wl.q(b).to(torch.float64).numpy()
        if fp8:
            kc, vc = wl.kv_fp8(b)
            k, v = dequantize_kv(kc.numpy(), ks), dequantize_kv(vc.numpy(), vs)
        else:
            kt, vt = wl.kv(b)
            k, v = kt.to(torch.float64).numpy(), vt.to(torch.float64).numpy()
        out[b] = ref_attention(q, k, v, scale, causal=True)
    return out
