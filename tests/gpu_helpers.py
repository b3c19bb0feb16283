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


LOG2E = 1.4426950408889634
KERNEL_CHUNK = 64          # keys per online-softmax step of the split-KV kernels
KERNEL_SLACK_LOG2 = 8.0    # the kernels move their reference maximum only past this margin


def rescale_replay(q_rows, k, kv_begin, kv_end, vis_end, scale, chunk=KERNEL_CHUNK, slack=KERNEL_SLACK_LOG2):
    """Replay, on the host, the split-KV kernels' lazy online-softmax rule for one segment, to show
    that a test input drives the branch that rescales the accumulators from a finite reference.

    The kernels walk the keys [kv_begin, kv_end) in chunks aligned to multiples of `chunk` and keep,
    per (query row, query head) column, a reference maximum m_ref (log2 units, -inf at first): a
    chunk whose largest visible score exceeds m_ref + slack moves m_ref to it and rescales o and l
    by 2^(old - new).  q_rows [R, Hq, D] and k [L, Hkv, D] are float64 (k dequantised for an 8-bit
    cache), vis_end [R] the exclusive causal key end of each row.

    Returns (finite, first, frac): finite [R, Hq] counts of rescales from a finite m_ref, first
    [R, Hq] counts of moves from -inf, and frac, the largest share of a column's final sum that
    came before one of its finite rescales (how much a wrong rescale factor would move the result)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, Hq, D = q_rows.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    c0 = (kv_begin // chunk) * chunk
    n = max(0, kv_end - c0)
    nch = -(-n // chunk)
    finite = np.zeros((R, Hq), dtype=np.int64)
    first = np.zeros((R, Hq), dtype=np.int64)
    frac = 0.0
    if nch == 0:
        return finite, first, frac
    pos = c0 + np.arange(nch * chunk)
    for g in range(Hkv):
        kg = np.zeros((nch * chunk, D))
        kg[:n] = k[c0:kv_end, g]
        s = scale * LOG2E * np.einsum("rhd,td->rht", q_rows[:, g * group:(g + 1) * group], kg)
        visible = (pos[None, :] >= kv_begin) & (pos[None, :] < np.minimum(kv_end, np.asarray(vis_end))[:, None])
        s = np.where(visible[:, None, :], s, -np.inf).reshape(R, group, nch, chunk)
        cmax = s.max(axis=3)                                          # [R, group, nch]
        top = cmax.max(axis=2, keepdims=True)
        safe = np.where(np.isfinite(top), top, 0.0)
        mass = np.where(np.isfinite(s), np.exp2(s - safe[..., None]), 0.0).sum(axis=3)   # [R, group, nch]
        total = mass.sum(axis=2)
        before = np.cumsum(mass, axis=2) - mass
        m_ref = np.full((R, group), -np.inf)
        for i in range(nch):
            need = cmax[:, :, i] > m_ref + slack
            fin = need & np.isfinite(m_ref)
            finite[:, g * group:(g + 1) * group] += fin
            first[:, g * group:(g + 1) * group] += need & ~np.isfinite(m_ref)
            if fin.any():
                frac = max(frac, float(np.max(np.where(fin & (total > 0), before[:, :, i] / np.where(total > 0, total, 1), 0))))
            m_ref = np.where(need, cmax[:, :, i], m_ref)
    return finite, first, frac
