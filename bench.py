#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one pass of the whole hot path for one layer: the split-KV kernel over the work map and
the combine kernel, with the map already on the device (it is built once per inference step and
shared by all layers).  Default workload: the mixed-length batch - 40 requests, 8 each at KV
lengths 1K, 4K, 16K, 64K and 128K tokens, one query token each, 64 query / 8 KV heads, head dim
128, bf16, 64-token pages in a shuffled block table, 512-token tiles.

Prints one JSON line: whole-step throughput in TB/s of algorithmic bytes (KV + Q + fp32 output +
block table + lengths), the split-KV kernel's roofline fraction, the fp64 CPU oracle timed on a
bounded sample, the static split-KV baseline and the per-CU busy spread.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "mixed-length GQA decode attention: achieved HBM TB/s (% peak) and µs/step"
PEAK_HBM_GBS = 8000.0
DESCRIPTIONS = {
    "mixed": "mixed-length decode: B=40, 8 each of KV 1K/4K/16K/64K/128K (shuffled), 1 query token, "
             "GQA 64q/8kv, d=128, bf16, paged 64-token KV (shuffled block table), tile 512",
    "uniform": "uniform decode: B=64 x KV 8192, 1 query token, GQA 64q/8kv, d=128, bf16, paged 64-token KV "
               "(shuffled block table), tile 512",
    "long_tail": "single long request plus short tail: KV 192K + 15 x U[1K,2K], 1 query token, GQA 64q/8kv, "
                 "d=128, bf16, paged 64-token KV (shuffled block table), tile 512",
    "control": "even control for the mixed batch: B=40 x KV 43622 (the mixed batch's tokens), 1 query token, "
               "GQA 64q/8kv, d=128, bf16, paged 64-token KV (shuffled block table), tile 512",
    "tiny": "worked example: KV 1024/5120/2048, 1 query token, GQA 64q/8kv, d=128, bf16, contiguous pages, "
            "tile 512, 4 workers",
    "mixed_tp8": "one GPU's share of the mixed batch under 8-way KV-head sharding: B=40, 8 each of KV "
                 "1K/4K/16K/64K/128K (shuffled), 1 query token, 8q/1kv, d=128, bf16, paged 64-token KV "
                 "(shuffled block table), tile 512",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(wl, page: int, kv_elem: int = 2) -> dict:
    """Bytes the step must move: K and V (kv_elem bytes per element; an 8-bit cache adds its
    per-head scales), Q, the fp32 output, the block table and the lengths."""
    tokens = sum(wl.kv_lens)
    pages = sum(-(-L // page) for L in wl.kv_lens)
    kv = tokens * wl.hkv * wl.head_dim * kv_elem * 2 + (2 * wl.hkv * 4 if kv_elem == 1 else 0)
    q = wl.batch * wl.hq * wl.head_dim * 2
    out = wl.batch * wl.hq * wl.head_dim * 4
    table = pages * 4
    lens = wl.batch * 4
    return {"kv": kv, "q": q, "out": out, "block_table": table, "seq_lens": lens,
            "step": kv + q + out + table + lens, "splitkv": kv + q + table + lens}


def per_cu_busy(timing) -> dict:
    """Union of [start, end) per compute unit (HW_ID CU/SH/SE fields + XCC_ID)."""
    import numpy as np
    t = timing.cpu().numpy().astype(np.int64)
    hw = t[:, 2]
    key = (t[:, 3] & 0xF) * 4096 + ((hw >> 13) & 0x7) * 512 + ((hw >> 12) & 1) * 256 + ((hw >> 8) & 0xF)
    busy = {}
    for k in np.unique(key):
        iv = sorted(zip(t[key == k, 0].tolist(), t[key == k, 1].tolist()))
        total, cs, ce = 0, iv[0][0], iv[0][1]
        for s, e in iv[1:]:
            if s > ce:
                total += ce - cs
                cs, ce = s, e
            else:
                ce = max(ce, e)
        total += ce - cs
        busy[int(k)] = total
    vals = np.array(list(busy.values()), dtype=np.float64)
    span = float(t[:, 1].max() - t[:, 0].min())
    return {"cus_seen": int(len(vals)), "max_over_mean": float(vals.max() / vals.mean()),
            "tail_fraction": float((vals.max() - vals.mean()) / vals.max()),
            "mean_busy_over_span": float(vals.mean() / span), "workgroups": int(t.shape[0])}


WARM_SECONDS = 0.05


def time_steps(fn_split, fn_combine, steps: int, warmup: int):
    """Two timed passes on the launch stream: (1) `steps` back-to-back steps bracketed by one event
    pair (the step rate); (2) the same steps with an event pair around every split-KV launch and
    every combine launch (per-kernel durations)."""
    import torch
    for i in range(warmup):
        fn_split(i)
        fn_combine(i)
    torch.cuda.synchronize()
    # untimed warmup also lasts at least WARM_SECONDS of device work: after a pause (cache packing
    # between sections) a few steps leave the clocks low for the start of the timed pass
    t_warm = time.perf_counter() + WARM_SECONDS
    i = warmup
    while time.perf_counter() < t_warm:
        for _ in range(4):
            fn_split(i)
            fn_combine(i)
            i += 1
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        fn_split(i)
        fn_combine(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        a, b, c, d = ev[i]
        a.record()
        fn_split(i)
        b.record()
        c.record()
        fn_combine(i)
        d.record()
    torch.cuda.synchronize()
    return {"total_ms": t0.elapsed_time(t1), "wall_s": wall,
            "split_ms": [a.elapsed_time(b) for a, b, _, _ in ev],
            "combine_ms": [c.elapsed_time(d) for _, _, c, d in ev]}


def kernel_source_digest(family: str = "decode") -> str:
    from load_balanced_split_attn_amd.record_traffic import kernel_source_digest as digest
    return digest(family)


def recorded_traffic(kernel: str, workload: str, family: str = "decode"):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs, if they were taken on
    the current kernel source (None otherwise)."""
    path = os.path.join(ROOT, "load_balanced_split_attn_amd", "measured_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel, {}).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != kernel_source_digest(family):
        return None
    return rec.get("bytes_per_launch")


def calibration_copy(dev) -> None:
    """A plain 1 GiB device-to-device copy (torch's copy kernel): the known-size reference that
    scales the FETCH_SIZE / WRITE_SIZE counters in the profile runs."""
    import torch
    src = torch.ones(2**30 // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_oracle_baseline(wl, budget_s: float, scale: float, workers: int, tile: int) -> dict:
    import numpy as np
    import torch
    from oracle.attention import ref_attention
    from oracle.plan import ref_plan
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    q = wl.q().to(torch.float64).numpy()
    # one pass over the batch's requests, each request's oracle call repeated so that the pass takes
    # about the time budget: before each request the repeat count is set from the rate measured so
    # far and the budget and tokens left; input generation and the bf16 -> fp64 widening are done
    # once per request and not timed
    left_tokens = sum(wl.kv_lens)
    spent, tokens, runs, reps_used = 0.0, 0, 0, []
    for b in range(wl.batch):
        k, v = wl.kv(b)
        kd, vd = k.to(torch.float64).numpy(), v.to(torch.float64).numpy()
        if b == 0:
            ref_attention(q[b:b + 1], kd, vd, scale)   # untimed warm-up (library and page faults)
        reps = 1
        if tokens > 0 and left_tokens > 0:
            rate = spent / tokens
            reps = max(1, int(round((budget_s - spent) / max(rate * left_tokens, 1e-9))))
        for _ in range(reps):
            t = time.perf_counter()
            ref_attention(q[b:b + 1], kd, vd, scale)
            spent += time.perf_counter() - t
            tokens += wl.kv_lens[b]
            runs += 1
        reps_used.append(reps)
        left_tokens -= wl.kv_lens[b]
        del kd, vd
    kv_bytes = tokens * wl.hkv * wl.head_dim * 2 * 2
    # the oracle's planner (pure Python) on the same batch, beside the library's host planner
    t = time.perf_counter()
    for _ in range(5):
        ref_plan(wl.kv_lens, workers, tile)
    ref_plan_us = (time.perf_counter() - t) / 5 * 1e6
    return {"value": kv_bytes / spent / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
            "ref_plan_us": round(ref_plan_us, 1),
            "sample": f"fp64 oracle (numpy) over all {wl.batch} requests of the same batch, each run "
                      f"{min(reps_used)}-{max(reps_used)} times ({runs} runs, {tokens} KV tokens), {spent:.1f} s of "
                      f"CPU time; bf16 KV bytes / time",
            "seconds": spent, "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count()}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


PEAK_BF16_TFLOPS = 2500.0


def prefill_flops(wl) -> int:
    """Algorithmic flops of causal chunked prefill: 4 * D * Hq per (row, visible key) pair."""
    total = 0
    for ql, kl in zip(wl.q_lens, wl.kv_lens):
        prefix = kl - ql
        total += ql * prefix + ql * (ql + 1) // 2
    return 4 * wl.head_dim * wl.hq * total


PV_LABELS = {None: "fp16 P.V (V*2^6, P*2^-6) on checked V chunks, bf16 hi+lo P for chunks fp16 does not hold "
                   "(default; V exact)",
             True: "bf16 V, P as bf16 hi+lo (every chunk)", False: "fp16 V and P, unchecked (V range-limited)"}


def prefill_unique_bytes(wl, segments: int, q_tile: int) -> int:
    """Bytes a prefill launch must move at least: Q, every request's K and V once, the partial slots
    written (m, l and 128 output values per (row, query head), fp32)."""
    rows = sum(wl.q_lens)
    q_bytes = rows * wl.hq * wl.head_dim * 2
    kv_bytes = sum(wl.kv_lens) * wl.hkv * wl.head_dim * 2 * 2
    part_bytes = segments * q_tile * wl.hq * (wl.head_dim + 2) * 4
    return q_bytes + kv_bytes + part_bytes


def optional_section(name: str, fn):
    """Run a comparison section that the headline does not depend on; a Python error in it (say, a
    device partitioned into fewer XCDs than the rated map assumes) is recorded in the line instead
    of ending the run."""
    try:
        return fn()
    except Exception as e:   # noqa: BLE001 - recorded in the output, never silent
        log(f"{name}: skipped ({type(e).__name__}: {e})")
        return {"error": f"{type(e).__name__}: {e}"}


def mfma_ceiling(dev, prefill_tflops: float) -> dict:
    """The bf16 rate this device's matrix cores sustain, measured beside the prefill kernel: the
    register-only probe (v_mfma_f32_16x16x32_bf16 flat out, 1,024 workgroups of four waves, eight
    launches back to back after two) and a library GEMM (torch.mm, 16384^3 bf16, A . B^T)."""
    import torch

    import load_balanced_split_attn_amd as lb

    def timed(fn, reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        work = sum(fn() for _ in range(reps))
        e1.record()
        torch.cuda.synchronize()
        return work / (e0.elapsed_time(e1) * 1e-3) / 1e12

    blocks, iters = 1024, 32768
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device=dev)
    probe = lambda: lb.attn_probe_mfma_rate(iters, blocks, sink)
    timed(probe, 2)
    probe_tf = timed(probe, 8)
    # the library's fastest square case on this device: A . B^T with both operands row-major
    # (~1.6 PFLOP/s at 16384^3, against ~1.37 for A . B)
    n = 16384
    g = torch.Generator(device=dev).manual_seed(5)
    a = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)

    def gemm():
        torch.mm(a, b.t(), out=c)
        return 2 * n ** 3

    timed(gemm, 3)
    gemm_tf = timed(gemm, 10)
    del a, b, c
    torch.cuda.empty_cache()
    # 16 cycles per 16x16x32 product on each of the 1,024 SIMDs: 1,048,576 flops per clock
    clock = probe_tf * 1e12 / (1024 * 1024) / 1e9
    log(f"matrix cores: probe {probe_tf:.0f} TFLOP/s (~{clock:.2f} GHz), library GEMM {gemm_tf:.0f} TFLOP/s")
    return {"probe_tflops": round(probe_tf, 1), "probe_implied_clock_GHz": round(clock, 3),
            "probe": f"v_mfma_f32_16x16x32_bf16 on register operands, {blocks} x 4 waves x {iters} x 8 products",
            "library_gemm_tflops": round(gemm_tf, 1), "library_gemm": f"torch.mm bf16 {n}x{n}x{n}, A . B^T",
            "prefill_frac_of_probe": round(prefill_tflops / probe_tf, 4),
            "prefill_frac_of_library_gemm": round(prefill_tflops / gemm_tf, 4)}


def bench_prefill(dev, workers_list, steps: int, warmup: int, q_tiles=(128, 256), exact_modes=(None, True, False)) -> dict:
    """Chunked prefill over cached prefixes: 8 requests x 2048-row causal chunks after prefixes drawn
    log-uniform in [8K, 128K]; q tiles of 128 or 256 rows x KV tiles of 512 on the same greedy
    planner; P.V in the default checked mode, exact on bf16 V, or on the unchecked fp16 path.  The
    section's roofline is the configuration as stated (128-row q tiles, default P.V)."""
    import numpy as np
    import torch

    import workloads as WL
    from load_balanced_split_attn_amd.paged import pack_paged
    from load_balanced_split_attn_amd.prefill import PrefillStep
    wl = WL.prefill()
    scale = 1.0 / math.sqrt(wl.head_dim)
    q = torch.cat([wl.q(b) for b in range(wl.batch)], dim=0).to(dev)
    kc, vc, bt = pack_paged(wl.kv, wl.kv_lens, 64, wl.hkv, wl.head_dim, wl.page_permutation, dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    flops = prefill_flops(wl)
    rows = []
    for q_tile in q_tiles:
        for exact in exact_modes:
            pv = PV_LABELS[exact]
            for W in workers_list:
                st = PrefillStep(wl.q_lens, wl.kv_lens, dev, num_workers=W, q_tile=q_tile, exact_pv=exact)
                r = time_steps(lambda i, st=st: st.splitkv(q, kc, vc, bt, scale), lambda i, st=st: st.combine(out),
                               steps, warmup)
                split_ms = float(np.mean(r["split_ms"]))
                tf = flops / (split_ms * 1e-3) / 1e12
                rows.append({"q_tile": q_tile, "pv": pv, "exact_pv": exact, "workers": W, "segments": st.S,
                             "us_per_step": round(r["total_ms"] / steps * 1e3, 1),
                             "splitkv_us": round(split_ms * 1e3, 1),
                             "combine_us": round(float(np.mean(r["combine_ms"])) * 1e3, 1),
                             "splitkv_tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
                log(f"prefill q_tile={q_tile} {'checked' if exact is None else ('exact' if exact else 'fp16')} W={W}: "
                    f"splitkv {split_ms * 1e3:.0f} us "
                    f"({rows[-1]['splitkv_tflops']} TFLOP/s)")
                del st
    prefix = wl.meta["prefix"]
    cached = sum(prefix) / sum(wl.kv_lens)

    def pick(q_tile, exact):
        cand = [x for x in rows if x["q_tile"] == q_tile and x["exact_pv"] == exact]
        return min(cand, key=lambda x: x["us_per_step"]) if cand else None

    stated = pick(128, None) or min(rows, key=lambda x: x["us_per_step"])
    fastest = min(rows, key=lambda x: x["us_per_step"])
    return {"workload": "chunked prefill: 8 x 2048-row causal chunks after prefixes log-uniform in [8K, 128K] "
                        f"({prefix}), GQA 64q/8kv, d=128, bf16 Q/K/V, q tile {stated['q_tile']} x KV tile 512, "
                        f"P.V: {stated['pv']}",
            "cached_fraction": round(cached, 4), "flops_per_step": flops,
            "us_per_step": stated["us_per_step"],
            "tflops_per_step": round(flops / (stated["us_per_step"] * 1e-6) / 1e12, 1),
            "roofline": {"bound": "mfma", "kernel": "splitkv_prefill_kernel", "dtype": "bf16",
                         "achieved": stated["splitkv_tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(stated["splitkv_tflops"] / PEAK_BF16_TFLOPS, 4),
                         # HBM bytes per launch from the counter runs (128-row units, checked P.V,
                         # 64 workers, on this kernel source), beside the bytes read or written once
                         "traffic": (recorded_traffic("splitkv_prefill_kernel", "chunked_q128_checked", "prefill")
                                     if (stated["q_tile"], stated["exact_pv"], stated["workers"]) == (128, None, 64)
                                     else None),
                         "unique_bytes": prefill_unique_bytes(wl, stated["segments"], stated["q_tile"])},
            "fastest": {k: fastest[k] for k in ("q_tile", "pv", "workers", "us_per_step", "splitkv_us",
                                                 "splitkv_tflops", "frac_of_bf16_peak")},
            "mfma_ceiling": optional_section("mfma_ceiling", lambda: mfma_ceiling(dev, stated["splitkv_tflops"])),
            "sweep": rows}


def claim_sweep(dev, wl, q, caches, bt, out, args, base_us: float) -> dict:
    """Run-time claiming (attn_splitkv_claimed) beside the static launch: one resident wave per SIMD
    (one-wave workgroups) takes the (list, KV head) items of maps with m times the resident lists,
    at 512- and 128-token tiles; beside each, the static launch over the same map (one workgroup per
    item, the hardware dispatcher placing them).  speedup = the default static step / this step."""
    import numpy as np
    import torch

    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.decode import DecodeStep
    scale = 1.0 / math.sqrt(wl.head_dim)
    copies = len(caches)
    kc, vc = caches[0]
    resident = lb.attn_query_workers(0, 8) * 8          # one wave per SIMD
    base_lists = resident // wl.hkv
    rows = []
    for mult in (1, 2, 4):
        for tile in (512, 128):
            for mode in ("claimed", "static"):
                if mode == "static" and mult == 1 and tile == 512:
                    continue   # the default launch itself
                st = DecodeStep(wl.kv_lens, dev, num_q_heads=wl.hq, num_workers=base_lists * mult, tile=tile,
                                head_groups=wl.hkv, resident_workgroups=resident if mode == "claimed" else None)

                def split(i, st=st):
                    k_, v_ = caches[i % copies]
                    st.splitkv(q, k_, v_, bt, scale)

                r = time_steps(split, lambda i, st=st: st.combine(out), args.static_steps, 2)
                us = r["total_ms"] / args.static_steps * 1e3
                n_wg = resident if mode == "claimed" else st.W * wl.hkv
                timing = torch.zeros((n_wg, 4), dtype=torch.int64, device=dev)
                st.splitkv(q, kc, vc, bt, scale, timing=timing)
                torch.cuda.synchronize()
                rows.append({"mode": mode, "lists": st.W, "tile": tile, "segments": st.S, "workgroups": n_wg,
                             "us_per_step": round(us, 2), "splitkv_us": round(float(np.mean(r["split_ms"])) * 1e3, 2),
                             "per_cu_max_over_mean": round(per_cu_busy(timing)["max_over_mean"], 3),
                             "speedup": round(base_us / us, 3)})
                log(f"{wl.name} {mode} lists={st.W} tile={tile}: {us:.1f} us")
                del st
    best = min(rows, key=lambda x: x["us_per_step"])
    return {"resident_workgroups": resident, "default_us": round(base_us, 2), "best": best, "sweep": rows}


def rated_compare(dev, wl, base, q, caches, bt, out, args, base_us: float, split_bytes: int,
                  kv_scales=None) -> dict:
    """The rate-proportional map beside the default (equal-budget) one, on the same workers: per-XCD
    rates from the default launch's own timestamps (calibrate_xcd_rates: three instrumented launches,
    every XCD running one head group of every list), then attn_plan_rated with worker w at the rate
    of XCD w mod 8 (a version-3 map: list-major launch, every workgroup of list w on XCD w mod 8), at
    the default tile and at 128-token tiles (short lists need the finer steps).  Beside them, equal
    rates in the same list-major order (the order alone) and the equal-budget map at 128-token tiles
    (the tile alone).  speedup = default step / this step."""
    import numpy as np
    import torch

    from load_balanced_split_attn_amd.decode import DecodeStep, calibrate_xcd_rates
    scale = 1.0 / math.sqrt(wl.head_dim)
    kc, vc = caches[0]
    copies = len(caches)
    G = base.head_groups
    rates = calibrate_xcd_rates(base, q, kc, vc, bt, scale, kv_scales=kv_scales)
    rows = []
    for label, tile, r in (("list-major, equal rates", base.tile, [1] * 8),
                           ("list-major, calibrated rates", base.tile, rates),
                           ("equal budgets, 128-token tiles", 128, None),
                           ("list-major, calibrated rates, 128-token tiles", 128, rates)):
        kw = dict(planner="rated", xcd_rates=r) if r is not None else {}
        st = DecodeStep(wl.kv_lens, dev, num_q_heads=wl.hq, num_workers=base.W, tile=tile, head_groups=G,
                        kv_dtype=base.kv_dtype, **kw)

        def split(i, st=st):
            k_, v_ = caches[i % copies]
            st.splitkv(q, k_, v_, bt, scale, kv_scales=kv_scales)

        rs = time_steps(split, lambda i, st=st: st.combine(out), args.steps, args.warmup)
        us = rs["total_ms"] / args.steps * 1e3
        split_us = float(np.mean(rs["split_ms"])) * 1e3
        timing = torch.zeros((st.W * G, 4), dtype=torch.int64, device=dev)
        st.splitkv(q, kc, vc, bt, scale, timing=timing, kv_scales=kv_scales)
        torch.cuda.synchronize()
        rows.append({"map": label, "tile": tile, "segments": st.S, "us_per_step": round(us, 2),
                     "splitkv_us": round(split_us, 2),
                     "splitkv_frac_hbm": round(split_bytes / (split_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "per_cu_max_over_mean": round(per_cu_busy(timing)["max_over_mean"], 3),
                     "speedup": round(base_us / us, 4)})
        log(f"{wl.name} {label}: {us:.1f} us/step vs {base_us:.1f} default")
        del st
    return {"what": "rate-proportional map (attn_plan_rated, version 3: list-major launch) against the "
                    "default equal-budget map on the same workers and tile",
            "xcd_rates": rates, "default_us": round(base_us, 2), "sweep": rows}


def bench_decode_leg(dev, name: str, args) -> dict:
    """Another decode batch timed the way the headline batch is: split-KV + combine per step on the
    dynamic map, the split-KV kernel's roofline fraction, per-CU busy max/mean (median of five
    instrumented launches, with their range), and the static split-KV baseline (plain and best S)."""
    import numpy as np
    import torch

    import load_balanced_split_attn_amd as lb
    import workloads as WL
    from load_balanced_split_attn_amd.decode import DecodeStep
    from load_balanced_split_attn_amd.paged import pack_paged
    wl = WL.BY_NAME[name]()
    page = 64
    scale = 1.0 / math.sqrt(wl.head_dim)
    nb = algorithmic_bytes(wl, page)
    q = wl.q().to(dev)
    kc, vc, bt = pack_paged(wl.kv, wl.kv_lens, page, wl.hkv, wl.head_dim, wl.page_permutation, dev)
    copies = 1 if nb["kv"] >= 2e9 else min(8, int(math.ceil(2e9 / max(nb["kv"], 1))))
    caches = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(copies - 1)]
    # one wave per (list, KV head) workgroup and one resident wave per SIMD: G = Hkv head groups
    G = min(args.head_groups, wl.hkv)
    workers = args.workers or lb.attn_query_workers(0, 8) * 8 // wl.hkv
    out = torch.empty((wl.batch, wl.hq, wl.head_dim), dtype=torch.float32, device=dev)

    def run(step, steps, warmup):
        def split(i):
            k_, v_ = caches[i % copies]
            step.splitkv(q, k_, v_, bt, scale)
        return time_steps(split, lambda i: step.combine(out), steps, warmup)

    def busy(step, n):
        vals = []
        for _ in range(n):
            timing = torch.zeros((step.W * G, 4), dtype=torch.int64, device=dev)
            step.splitkv(q, kc, vc, bt, scale, timing=timing)
            torch.cuda.synchronize()
            vals.append(per_cu_busy(timing)["max_over_mean"])
        return vals

    step = DecodeStep(wl.kv_lens, dev, num_q_heads=wl.hq, num_workers=workers, tile=args.tile, head_groups=G,
                      launch_order=args.launch_order)
    r = run(step, args.steps, args.warmup)
    ms = r["total_ms"] / args.steps
    split_ms = float(np.mean(r["split_ms"]))
    achieved = nb["splitkv"] / (split_ms * 1e-3) / 1e9
    spread = busy(step, 5)
    max_tiles = max(-(-L // args.tile) for L in wl.kv_lens)
    plain = min(max(1, -(-step.W // wl.batch)), max_tiles)
    rows = []
    for S in sorted(set([plain] + [x for x in (1, 2, 4, 8, 16, 32, 64) if x <= max_tiles])):
        st = DecodeStep(wl.kv_lens, dev, num_q_heads=wl.hq, tile=args.tile, head_groups=G, static_splits=S)
        rs = run(st, args.static_steps, 2)
        rows.append({"splits": S, "workgroups": st.W * G,
                     "us_per_step": round(rs["total_ms"] / args.static_steps * 1e3, 2),
                     "per_cu_max_over_mean": round(float(np.median(busy(st, 1))), 3)})
        del st
    best = min(rows, key=lambda x: x["us_per_step"])
    plain_row = next(x for x in rows if x["splits"] == plain)
    log(f"{name}: step {ms * 1e3:.1f} us, splitkv {split_ms * 1e3:.1f} us ({achieved:.0f} GB/s), per-CU "
        f"max/mean {np.median(spread):.3f}; static plain S={plain} {plain_row['us_per_step']} us, best "
        f"S={best['splits']} {best['us_per_step']} us")
    res = {"workload": DESCRIPTIONS[name], "us_per_step": round(ms * 1e3, 2),
           "value": round(nb["step"] / (ms * 1e-3) / 1e12, 4), "unit": "TB/s",
           "workers": step.W, "segments": step.S, "tiles": step.T, "cache_copies": copies,
           "roofline": {"bound": "hbm", "kernel": "splitkv_decode_kernel", "achieved": round(achieved, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                        "bytes_per_launch": nb["splitkv"], "avg_launch_us": round(split_ms * 1e3, 2)},
           "combine_us": round(float(np.mean(r["combine_ms"])) * 1e3, 2),
           "per_cu_busy": {"max_over_mean": round(float(np.median(spread)), 3),
                           "range_of_5": [round(min(spread), 3), round(max(spread), 3)]},
           "static_baseline": {"plain_splits": plain, "plain_us": plain_row["us_per_step"],
                               "best_splits": best["splits"], "best_us": best["us_per_step"],
                               "speedup_vs_plain": round(plain_row["us_per_step"] / (ms * 1e3), 3),
                               "speedup_vs_best": round(best["us_per_step"] / (ms * 1e3), 3), "sweep": rows}}
    if not args.no_claim:
        res["claimed"] = claim_sweep(dev, wl, q, caches, bt, out, args, ms * 1e3)
    if not args.no_rated:
        res["xcd_rated"] = optional_section(
            "xcd_rated", lambda: rated_compare(dev, wl, step, q, caches, bt, out, args, ms * 1e3, nb["splitkv"]))
    del caches, kc, vc, step
    torch.cuda.empty_cache()
    return res


def bench_fp8(dev, wl, args, bf16_us: float) -> dict:
    """The same decode step over an 8-bit (E4M3) KV cache with per-head scales: the same map shape
    and combine, half the KV bytes."""
    import numpy as np
    import torch

    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.decode import DecodeStep
    from load_balanced_split_attn_amd.paged import pack_paged
    page = 64
    scale = 1.0 / math.sqrt(wl.head_dim)
    q = wl.q().to(dev)
    kc, vc, bt = pack_paged(wl.kv_fp8, wl.kv_lens, page, wl.hkv, wl.head_dim, wl.page_permutation, dev,
                            dtype=torch.uint8)
    ks, vs = (s.to(dev) for s in wl.kv_scales())
    nb = algorithmic_bytes(wl, page, kv_elem=1)
    copies = 1 if nb["kv"] >= 2e9 else min(8, int(math.ceil(2e9 / max(nb["kv"], 1))))
    caches = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(copies - 1)]
    workers = args.workers or (wl.workers if wl.workers else
                               lb.attn_query_workers(0, args.head_groups, lb.KV_FP8_E4M3))
    step = DecodeStep(wl.kv_lens, dev, num_q_heads=wl.hq, num_workers=workers, tile=args.tile,
                      head_groups=args.head_groups,
                      kv_dtype=lb.KV_FP8_E4M3)
    out = torch.empty((wl.batch, wl.hq, wl.head_dim), dtype=torch.float32, device=dev)
    # the same map built on the device (attn_plan_device), timed with events on the stream
    lens_d = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    map_d = torch.zeros(lb.device_map_words(wl.batch, workers), dtype=torch.int32, device=dev)
    for _ in range(3):
        lb.attn_plan_device(lens_d, workers, args.tile, map_d)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        lb.attn_plan_device(lens_d, workers, args.tile, map_d)
    e1.record()
    torch.cuda.synchronize()
    plan_device_us = e0.elapsed_time(e1) / 20 * 1e3
    plan_device_exact = bool(np.array_equal(map_d.cpu().numpy()[:len(step.map_host)], step.map_host))

    def split(i):
        k_, v_ = caches[i % copies]
        step.splitkv(q, k_, v_, bt, scale, kv_scales=(ks, vs))

    r = time_steps(split, lambda i: step.combine(out), args.steps, args.warmup)
    ms = r["total_ms"] / args.steps
    split_ms = float(np.mean(r["split_ms"]))
    achieved = nb["splitkv"] / (split_ms * 1e-3) / 1e9
    timing = torch.zeros((step.W * args.head_groups, 4), dtype=torch.int64, device=dev)
    step.splitkv(q, kc, vc, bt, scale, timing=timing, kv_scales=(ks, vs))
    torch.cuda.synchronize()
    log(f"fp8 cache: step {ms * 1e3:.1f} us, splitkv {split_ms * 1e3:.1f} us ({achieved:.0f} GB/s)")
    rated = None
    if not args.no_rated and wl.name != "tiny":
        rated = optional_section("xcd_rated", lambda: rated_compare(dev, wl, step, q, caches, bt, out, args, ms * 1e3,
                                                                    nb["splitkv"], kv_scales=(ks, vs)))
    res = {"workload": DESCRIPTIONS[wl.name].replace("bf16, paged", "bf16 q, E4M3 KV with per-head fp32 scales, "
                                                                     "paged"),
            "algorithmic_bytes": nb["step"], "us_per_step": round(ms * 1e3, 2),
            "value": round(nb["step"] / (ms * 1e-3) / 1e12, 4), "unit": "TB/s",
            "speedup_vs_bf16_step": round(bf16_us / (ms * 1e3), 3),
            "workers": step.W, "segments": step.S, "cache_copies": copies,
            "roofline": {"bound": "hbm", "kernel": "splitkv_decode_kernel<KvFp8>", "achieved": round(achieved, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "traffic": recorded_traffic("splitkv_decode_kernel_fp8", wl.name),
                         "bytes_per_launch": nb["splitkv"], "avg_launch_us": round(split_ms * 1e3, 2)},
            "combine_us": round(float(np.mean(r["combine_ms"])) * 1e3, 2),
            "per_cu_busy": per_cu_busy(timing)}
    if rated:
        res["xcd_rated"] = rated
    return res


def bench_mtp(dev, base: str, args, decode_us: float) -> dict:
    """Multi-token decode (verify step of multi-token prediction) over the same KV lengths: every
    request carries q_len = 2 or 4 query tokens, causal among themselves; bf16 and E4M3 caches."""
    import numpy as np
    import torch

    import load_balanced_split_attn_amd as lb
    import workloads as WL
    from load_balanced_split_attn_amd.mtp import MtpDecodeStep
    from load_balanced_split_attn_amd.paged import pack_paged
    page = 64
    scale = 1.0 / math.sqrt(128)
    src = WL.BY_NAME[base]()
    rows = []
    for fp8 in (False, True):
        if fp8:
            kc, vc, bt = pack_paged(src.kv_fp8, src.kv_lens, page, src.hkv, src.head_dim, src.page_permutation, dev,
                                    dtype=torch.uint8)
            scales = tuple(s.to(dev) for s in src.kv_scales())
        else:
            kc, vc, bt = pack_paged(src.kv, src.kv_lens, page, src.hkv, src.head_dim, src.page_permutation, dev)
            scales = None
        for q_len in ((2, 4) if not fp8 else (4,)):
            wl = WL.mtp(q_len, base)
            q = torch.cat([wl.q(b) for b in range(wl.batch)]).to(dev)
            kvd = lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16
            workers = args.workers or lb.attn_query_workers(0, args.head_groups, kvd)
            st = MtpDecodeStep(wl.q_lens, wl.kv_lens, dev, num_workers=workers, tile=args.tile,
                               head_groups=args.head_groups, kv_dtype=kvd)
            out = torch.empty(q.shape, dtype=torch.float32, device=dev)
            r = time_steps(lambda i: st.splitkv(q, kc, vc, bt, scale, kv_scales=scales), lambda i: st.combine(out),
                           args.steps, args.warmup)
            ms = r["total_ms"] / args.steps
            split_ms = float(np.mean(r["split_ms"]))
            nb = algorithmic_bytes(src, page, kv_elem=1 if fp8 else 2)
            n_rows = sum(wl.q_lens)
            step_bytes = nb["kv"] + nb["block_table"] + n_rows * wl.hq * wl.head_dim * (2 + 4) + 3 * wl.batch * 4
            rows.append({"kv": "e4m3" if fp8 else "bf16", "q_len": q_len, "query_tokens": n_rows,
                         "us_per_step": round(ms * 1e3, 2), "splitkv_us": round(split_ms * 1e3, 2),
                         "combine_us": round(float(np.mean(r["combine_ms"])) * 1e3, 2),
                         "TB_per_s": round(step_bytes / (ms * 1e-3) / 1e12, 4),
                         "splitkv_frac_hbm": round((step_bytes - n_rows * wl.hq * wl.head_dim * 4) /
                                                   (split_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
            log(f"mtp {rows[-1]['kv']} q_len={q_len}: step {ms * 1e3:.1f} us, splitkv {split_ms * 1e3:.1f} us")
            del st, q, out
        del kc, vc
        torch.cuda.empty_cache()
    return {"workload": f"multi-token decode over the {base} batch's KV lengths: q_len drafted tokens per "
                        "request (the last q_len positions, causal among themselves)",
            "decode_us_per_step": round(decode_us, 2), "sweep": rows}


def unfused_store_step(dev, hq: int, hkv: int, page: int, theta: float, eps: float):
    """The producer step as separate GPU tensor ops, the unfused form the fused kernel replaces:
    RMSNorm, RoPE (fp64 angles), Hadamard as a matrix product, rounding / E4M3 quantisation, and an
    index scatter into the blocked paged cache.  A measurement baseline only."""
    import math
    import torch
    import torch.nn.functional as F
    D = 128
    h = torch.ones((1, 1), dtype=torch.float32)
    while h.shape[0] < D:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    hmat = (h / math.sqrt(D)).to(dev)                       # symmetric: x @ H = H x
    freq = torch.tensor([theta ** (-2.0 * i / D) for i in range(D // 2)], dtype=torch.float64, device=dev)
    d = torch.arange(D, device=dev)
    heads = torch.arange(hkv, device=dev)

    def rope(x, cos, sin):
        x1, x2 = x[..., :D // 2], x[..., D // 2:]
        return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], -1)

    def step(q, k, v, pos, q_out, kc, vc, bt, qw, kw, scales):
        fp8 = kc.dtype == torch.uint8
        w = 64 if fp8 else 32
        qf = F.rms_norm(q.float(), (D,), qw, eps)
        kf = F.rms_norm(k.float(), (D,), kw, eps)
        ang = torch.remainder(pos.double()[:, None] * freq[None, :], 2 * math.pi)
        cos, sin = torch.cos(ang).float()[:, None, :], torch.sin(ang).float()[:, None, :]
        qf = rope(qf, cos, sin) @ hmat
        kf = rope(kf, cos, sin) @ hmat
        q_out.copy_(qf.to(torch.bfloat16))
        if fp8:
            ks, vs = scales
            kq = (kf / ks[None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
            vq = (v.float() / vs[None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            kq, vq = kf.to(torch.bfloat16), v
        p64 = pos.long()
        pid = bt.gather(1, (p64 // page)[:, None])[:, 0].long()
        t = p64 % page
        blk = ((pid[:, None] * hkv + heads[None, :]) * (page * D))[:, :, None]
        k_idx = blk + (((d // w) * page)[None, None, :] + t[:, None, None]) * w + (d % w)[None, None, :]
        v_idx = blk + ((t // w)[:, None, None] * D + d[None, None, :]) * w + (t % w)[:, None, None]
        kc.view(-1).index_copy_(0, k_idx.reshape(-1), kq.reshape(-1))
        vc.view(-1).index_copy_(0, v_idx.reshape(-1), vq.reshape(-1))

    return step


def bench_unfused_store(dev, wl, q, k, v, pos, bt, qw, kw, scales, q_ref, kc_ref, vc_ref, reps: int) -> dict:
    """Time the unfused producer step on the same inputs after checking it stores what the fused
    kernel stored (q within one bf16 step, cache bytes equal but for rounding ties); timed eagerly
    (launch by launch, as an unfused framework runs it) and as one HIP graph of `reps` calls, whose
    replays are checked against the eager result."""
    import torch
    step = unfused_store_step(dev, wl.hq, wl.hkv, 64, 10000.0, 1e-6)
    kc, vc, q_out = torch.zeros_like(kc_ref), torch.zeros_like(vc_ref), torch.empty_like(q_ref)
    f = lambda: step(q, k, v, pos, q_out, kc, vc, bt, qw, kw, scales)
    f()
    torch.cuda.synchronize()
    dq = (q_out.float() - q_ref.float()).abs()
    step_q = torch.ldexp(torch.ones_like(dq), torch.frexp(q_ref.float())[1] - 8)
    same = {"q_within_one_bf16_step": bool((dq <= step_q + 1e-6).all().item()),
            "k_bytes_equal": round(float((kc.view(torch.uint8) == kc_ref.view(torch.uint8)).float().mean().item()), 5),
            "v_bytes_equal": round(float((vc.view(torch.uint8) == vc_ref.view(torch.uint8)).float().mean().item()), 5)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        f()
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) / reps * 1e3
    # the same calls captured once and replayed; kept only if every replay reproduces the eager result
    graph_us = None
    kc_eager, vc_eager, q_eager = kc.clone(), vc.clone(), q_out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            f()
    ok = True
    for _ in range(3):
        kc.zero_()
        vc.zero_()
        q_out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ok &= bool(torch.equal(kc, kc_eager) and torch.equal(vc, vc_eager) and torch.equal(q_out, q_eager))
    if ok:
        e0.record()
        for _ in range(10):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = round(e0.elapsed_time(e1) / (10 * reps) * 1e3, 2)
    del graph
    return {"eager_us": round(eager_us, 2), "graph_us": graph_us, "graph_replays_match": ok, "matches_fused": same}


def bench_store_kv(dev, wl, args) -> dict:
    """The fused producer step (RMSNorm + RoPE + Hadamard on q and k, K/V stored into the blocked
    paged cache) for one decode step of the batch, and for a 4096-token step; bf16 and E4M3.  Each
    point is a HIP graph of 20 launches replayed back to back (the kernel, not the Python binding's
    per-call cost), timed with events on the replay stream."""
    import numpy as np
    import torch

    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.paged import cache_shapes, pages_for
    rows = []
    reps, replays = 20, 10
    for B, lens in ((wl.batch, list(wl.kv_lens)), (4096, [int(x) for x in np.random.default_rng(3).integers(
            0, 131072, size=4096)])):
        g = torch.Generator().manual_seed(B)
        q = torch.randn(B, wl.hq, wl.head_dim, generator=g).to(torch.bfloat16).to(dev)
        k = torch.randn(B, wl.hkv, wl.head_dim, generator=g).to(torch.bfloat16).to(dev)
        v = torch.randn(B, wl.hkv, wl.head_dim, generator=g).to(torch.bfloat16).to(dev)
        qw = torch.ones(wl.head_dim, device=dev)
        kw = torch.ones(wl.head_dim, device=dev)
        pos = torch.tensor(lens, dtype=torch.int32, device=dev)
        # one page per request around its new token is enough to receive the writes
        stride = max(pages_for(L + 1, 64) for L in lens)
        bt = torch.zeros((B, stride), dtype=torch.int32)
        for b, L in enumerate(lens):
            bt[b, L // 64] = b
        bt = bt.to(dev)
        q_out = torch.empty_like(q)
        for fp8 in (False, True):
            dtype = torch.uint8 if fp8 else torch.bfloat16
            ksh, vsh = cache_shapes(B, wl.hkv, 64, wl.head_dim, dtype)
            kc = torch.zeros(ksh, dtype=dtype, device=dev)
            vc = torch.zeros(vsh, dtype=dtype, device=dev)
            sc = (torch.full((wl.hkv,), 0.02, device=dev), torch.full((wl.hkv,), 0.02, device=dev)) if fp8 else None
            f = lambda: lb.attn_store_kv(q, k, v, pos, q_out, kc, vc, bt, q_norm_w=qw, k_norm_w=kw,
                                         rope_theta=10000.0, hadamard=True, kv_scales=sc)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(3):
                    f()
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(reps):
                    f()
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / (reps * replays) * 1e3
            unfused = (None if getattr(args, "no_unfused", False)
                       else bench_unfused_store(dev, wl, q, k, v, pos, bt, qw, kw, sc, q_out, kc, vc, reps))
            e = 1 if fp8 else 2
            nbytes = B * (wl.hq + 2 * wl.hkv) * wl.head_dim * 2 + B * wl.hq * wl.head_dim * 2 + \
                B * 2 * wl.hkv * wl.head_dim * e + B * 8 + 2 * wl.head_dim * 4
            # appending one token to the dim-major V tiles touches one 64-byte row per (dim, head)
            v_rows = B * wl.hkv * wl.head_dim * 64
            rows.append({"tokens": B, "kv": "e4m3" if fp8 else "bf16", "us": round(us, 2),
                         "algorithmic_bytes": nbytes, "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                         "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 8e12, 4), "v_rows_touched_bytes": v_rows,
                         "unfused": unfused,
                         "fused_speedup_graph": (round(unfused["graph_us"] / us, 2)
                                                 if unfused and unfused["graph_us"] else None)})
            log(f"store_kv B={B} {'e4m3' if fp8 else 'bf16'}: {us:.1f} us"
                + (f"; unfused ops: graph {unfused['graph_us']} us, eager {unfused['eager_us']} us" if unfused else ""))
            del graph, kc, vc
    return {"workload": "producer step: RMSNorm + RoPE + Hadamard on q and k, K/V stored in the blocked paged "
                        "cache, for the batch's new tokens and for a 4096-token step (each token its own page)",
            "timing": f"HIP graph of {reps} launches, {replays} replays, events on the replay stream",
            "bound": "latency at the batch's size; at 4096 tokens the one-token V append, which touches one "
                     "64-byte row per (dim, head)", "sweep": rows,
            "chunk": bench_store_chunk(dev, reps, replays)}


def _graph_us(f, reps: int, replays: int) -> float:
    """Average time of f() captured `reps` times in one HIP graph, replayed `replays` times."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            f()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            f()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / (reps * replays) * 1e3


def bench_store_chunk(dev, reps: int, replays: int) -> dict:
    """The producer step of a prefill chunk: the chunked-prefill batch's 8 x 2048 new tokens appended
    after their cached prefixes, by attn_store_kv_chunk (V in whole 64-byte rows) and, on the same
    tokens, by the one-token path (each token its own row of the block table)."""
    import torch

    import load_balanced_split_attn_amd as lb
    import workloads as WL
    from load_balanced_split_attn_amd.paged import cache_shapes
    pw = WL.prefill()
    n, prefix = list(pw.q_lens), list(pw.meta["prefix"])
    B, rows_n, hq, hkv, D, page = len(n), sum(n), pw.hq, pw.hkv, pw.head_dim, 64
    first = [p // page for p in prefix]
    last = [(p + c - 1) // page for p, c in zip(prefix, n)]
    stride = max(last) + 1
    bt = torch.zeros((B, stride), dtype=torch.int32)
    pid = 0
    for b in range(B):
        for lp in range(first[b], last[b] + 1):
            bt[b, lp] = pid
            pid += 1
    num_pages = pid
    bt = bt.to(dev)
    g = torch.Generator().manual_seed(17)
    q = torch.randn(rows_n, hq, D, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(rows_n, hkv, D, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(rows_n, hkv, D, generator=g).to(torch.bfloat16).to(dev)
    qw = torch.ones(D, device=dev)
    kw = torch.ones(D, device=dev)
    q_lens = torch.tensor(n, dtype=torch.int32, device=dev)
    starts = [0]
    for c in n[:-1]:
        starts.append(starts[-1] + c)
    q_start = torch.tensor(starts, dtype=torch.int32, device=dev)
    pos0 = torch.tensor(prefix, dtype=torch.int32, device=dev)
    req = torch.repeat_interleave(torch.arange(B), torch.tensor(n))
    pos_rows = torch.tensor([prefix[b] + j for b in range(B) for j in range(n[b])], dtype=torch.int32, device=dev)
    bt_rows = bt[req.to(dev)].contiguous()
    q_out = torch.empty_like(q)
    out = []
    for fp8 in (False, True):
        dtype = torch.uint8 if fp8 else torch.bfloat16
        ksh, vsh = cache_shapes(num_pages, hkv, page, D, dtype)
        kc = torch.zeros(ksh, dtype=dtype, device=dev)
        vc = torch.zeros(vsh, dtype=dtype, device=dev)
        sc = (torch.full((hkv,), 0.02, device=dev), torch.full((hkv,), 0.02, device=dev)) if fp8 else None
        common = dict(q_norm_w=qw, k_norm_w=kw, rope_theta=10000.0, hadamard=True, kv_scales=sc)
        us_chunk = _graph_us(lambda: lb.attn_store_kv_chunk(q, k, v, q_lens, q_start, pos0, max(n), q_out, kc, vc, bt,
                                                            **common), reps, replays)
        us_token = _graph_us(lambda: lb.attn_store_kv(q, k, v, pos_rows, q_out, kc, vc, bt_rows, **common),
                             reps, replays)
        e = 1 if fp8 else 2
        nbytes = rows_n * (hq + 2 * hkv) * D * 2 + rows_n * hq * D * 2 + rows_n * 2 * hkv * D * e + 3 * B * 4 + \
            2 * D * 4 + sum(last[b] - first[b] + 1 for b in range(B)) * 4
        out.append({"kv": "e4m3" if fp8 else "bf16", "tokens": rows_n, "chunk_us": round(us_chunk, 2),
                    "one_token_path_us": round(us_token, 2), "speedup": round(us_token / us_chunk, 2),
                    "algorithmic_bytes": nbytes, "GB_per_s": round(nbytes / (us_chunk * 1e-6) / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / (us_chunk * 1e-6) / 8e12, 4)})
        log(f"store_kv chunk 8x2048 {'e4m3' if fp8 else 'bf16'}: chunk path {us_chunk:.1f} us, one-token path "
            f"{us_token:.1f} us")
        del kc, vc
    # the step reads and writes about equal bytes; a plain copy of half its bytes is the read+write
    # rate HBM gives such a mix
    ceiling = copy_ceiling(dev, out[0]["algorithmic_bytes"] // 2, reps, replays)
    for row in out:
        row["frac_of_copy_ceiling"] = round(row["GB_per_s"] / ceiling["GB_per_s"], 4)
    log(f"store_kv chunk: copy ceiling {ceiling['GB_per_s']:.0f} GB/s read + write")
    return {"workload": "producer step of a prefill chunk: the chunked-prefill batch's 8 x 2048 new tokens after "
                        f"their cached prefixes ({prefix}), 64 q / 8 kv heads, RMSNorm + RoPE + Hadamard",
            "sweep": out, "copy_ceiling": ceiling}


def copy_ceiling(dev, nbytes: int, reps: int, replays: int) -> dict:
    """Read + write rate of a plain device copy of nbytes (torch's copy kernel, a HIP graph of reps
    copies replayed): what HBM sustains for a kernel that reads and writes equal amounts."""
    import torch
    src = torch.ones(nbytes // 16 * 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    us = _graph_us(lambda: dst.copy_(src), reps, replays)
    moved = 2 * src.numel() * 4
    del src, dst
    return {"what": "torch copy_ of a device buffer, read + write bytes / time", "bytes_each_way": moved // 2,
            "us": round(us, 2), "GB_per_s": round(moved / (us * 1e-6) / 1e9, 1)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--workers", type=int, default=None, help="work lists (default: fill the device once)")
    ap.add_argument("--head-groups", type=int, default=8)
    ap.add_argument("--tile", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-static", action="store_true")
    ap.add_argument("--static-steps", type=int, default=10)
    ap.add_argument("--calibration-copy", action="store_true",
                    help="run one plain 1 GiB copy first (reference for the HBM byte counters)")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill report")
    ap.add_argument("--prefill-workers", default="64")
    ap.add_argument("--prefill-q-tiles", default="128,256", help="query rows per prefill unit (128 and/or 256)")
    ap.add_argument("--prefill-pv", default="checked,exact,fp16",
                    help="prefill P.V paths to time: checked (the default), exact and/or fp16")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--no-claim", action="store_true", help="skip the run-time claiming comparison")
    ap.add_argument("--no-rated", action="store_true", help="skip the rate-proportional map comparison")
    ap.add_argument("--launch-order", default="auto", choices=("auto", "head", "list"),
                    help="order of the decode steps' split-KV workgroups (DecodeStep's launch_order)")
    ap.add_argument("--legs", default="uniform,long_tail,mixed_tp8",
                    help="other decode batches timed beside the headline one (comma list, '' for none)")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the chunked-prefill report (profiling runs); prints its JSON")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 8-bit KV cache report")
    ap.add_argument("--no-mtp", action="store_true", help="skip the multi-token decode report")
    ap.add_argument("--no-store", action="store_true", help="skip the producer-step report")
    ap.add_argument("--only-store", action="store_true",
                    help="run only the producer-step report on --workload (profiling runs); prints its JSON")
    ap.add_argument("--no-unfused", action="store_true",
                    help="producer-step report without the separate-tensor-ops comparison (counter runs)")
    ap.add_argument("--only-store-chunk", action="store_true",
                    help="run only the prefill-chunk producer-step report (profiling runs); prints its JSON")
    ap.add_argument("--only-fp8", action="store_true",
                    help="run only the 8-bit KV cache report on --workload (profiling runs); prints its JSON")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (decode attention shards by "
              "request or KV head with no exchange). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import load_balanced_split_attn_amd as lb
    import workloads as WL
    from load_balanced_split_attn_amd.decode import DecodeStep
    from load_balanced_split_attn_amd.paged import pack_paged

    lb.lib()
    dev = torch.device("cuda:0")
    if args.calibration_copy:
        calibration_copy(dev)
    prefill_args = ([int(x) for x in args.prefill_workers.split(",")], args.prefill_steps, 1,
                    tuple(int(x) for x in args.prefill_q_tiles.split(",")),
                    tuple({"checked": None, "exact": True, "fp16": False}[x.strip()] for x in args.prefill_pv.split(",")))
    if args.only_prefill:
        print(json.dumps(bench_prefill(dev, *prefill_args)), flush=True)
        return 0
    wl = WL.BY_NAME[args.workload]()
    if args.only_fp8:
        print(json.dumps(bench_fp8(dev, wl, args, float("nan"))), flush=True)
        return 0
    if args.only_store:
        print(json.dumps(bench_store_kv(dev, wl, args)), flush=True)
        return 0
    if args.only_store_chunk:
        print(json.dumps(bench_store_chunk(dev, 20, 10)), flush=True)
        return 0
    scale = 1.0 / math.sqrt(wl.head_dim)
    page = 64
    nbytes = algorithmic_bytes(wl, page)
    log(f"workload {wl.name}: B={wl.batch} tokens={sum(wl.kv_lens)} KV={nbytes['kv'] / 1e9:.2f} GB")

    t = time.perf_counter()
    q = wl.q().to(dev)
    kc, vc, bt = pack_paged(wl.kv, wl.kv_lens, page, wl.hkv, wl.head_dim, wl.page_permutation, dev)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.perf_counter() - t:.1f} s)")
    # below 2 GB of KV, rotate over copies so consecutive steps do not hit the 256 MB MALL
    copies = 1 if nbytes["kv"] >= 2e9 else min(8, int(math.ceil(2e9 / max(nbytes["kv"], 1))))
    caches = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(copies - 1)]

    workers = args.workers or (wl.workers if wl.workers else lb.attn_query_workers(0, args.head_groups))
    plan_t = time.perf_counter()
    step = DecodeStep(wl.kv_lens, dev, num_q_heads=wl.hq, num_workers=workers, tile=args.tile,
                      head_groups=args.head_groups, launch_order=args.launch_order)
    plan_s = time.perf_counter() - plan_t
    t = time.perf_counter()
    for _ in range(100):
        lb.attn_plan(wl.kv_lens, workers, args.tile)
    plan_us = (time.perf_counter() - t) / 100 * 1e6
    # the C planner alone (one ctypes call into a buffer of the right size), and the map's upload
    import ctypes
    lens_h = np.ascontiguousarray(np.asarray(wl.kv_lens, dtype=np.int32))
    buf = np.zeros(len(step.map_host), dtype=np.int32)
    i32p = ctypes.POINTER(ctypes.c_int32)
    words = ctypes.c_int32(0)
    fn, lens_p, buf_p, words_p = lb.lib().attn_plan, lens_h.ctypes.data_as(i32p), buf.ctypes.data_as(i32p), \
        ctypes.byref(words)
    n_lens, n_buf = len(lens_h), len(buf)
    t = time.perf_counter()
    for _ in range(1000):
        fn(lens_p, n_lens, workers, args.tile, buf_p, n_buf, words_p)
    plan_c_us = (time.perf_counter() - t) / 1000 * 1e6
    assert np.array_equal(buf, step.map_host)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(100):
        torch.from_numpy(buf).to(dev)
    torch.cuda.synchronize()
    upload_us = (time.perf_counter() - t) / 100 * 1e6
    out = torch.empty((wl.batch, wl.hq, wl.head_dim), dtype=torch.float32, device=dev)
    # the same map built on the device (attn_plan_device), timed with events on the stream
    lens_d = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    map_d = torch.zeros(lb.device_map_words(wl.batch, workers), dtype=torch.int32, device=dev)
    for _ in range(3):
        lb.attn_plan_device(lens_d, workers, args.tile, map_d)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        lb.attn_plan_device(lens_d, workers, args.tile, map_d)
    e1.record()
    torch.cuda.synchronize()
    plan_device_us = e0.elapsed_time(e1) / 20 * 1e3
    plan_device_exact = bool(np.array_equal(map_d.cpu().numpy()[:len(step.map_host)], step.map_host))

    def split(i):
        k_, v_ = caches[i % copies]
        step.splitkv(q, k_, v_, bt, scale)

    def comb(i):
        step.combine(out)

    log(f"dynamic map: W={step.W} G={args.head_groups} S={step.S} T={step.T}; timing {args.steps} steps")
    r = time_steps(split, comb, args.steps, args.warmup)
    ms_per_step = r["total_ms"] / args.steps
    split_ms = float(np.mean(r["split_ms"]))
    value = nbytes["step"] / (ms_per_step * 1e-3) / 1e12
    achieved = nbytes["splitkv"] / (split_ms * 1e-3) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us ({value:.3f} TB/s), splitkv {split_ms * 1e3:.1f} us ({achieved:.0f} GB/s)")

    result = {
        "metric": METRIC, "value": round(value, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[wl.name], "name": wl.name, "batch": wl.batch,
                   "kv_tokens": sum(wl.kv_lens), "q_heads": wl.hq, "kv_heads": wl.hkv, "head_dim": wl.head_dim,
                   "page": page, "tile": args.tile, "workers": step.W, "head_groups": args.head_groups,
                   "launch_order": "list-major" if step.list_major else "head-major",
                   "segments": step.S, "tiles": step.T, "cache_copies": copies},
        "us_per_step": round(ms_per_step * 1e3, 2),
        "splitkv_us_p10_p50_p90": [round(float(np.percentile(r["split_ms"], p)) * 1e3, 2) for p in (10, 50, 90)],
        "pct_peak_hbm": round(100 * value * 1e3 / PEAK_HBM_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": "splitkv_decode_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic("splitkv_decode_kernel", wl.name),
                     "bytes_per_launch": nbytes["splitkv"], "avg_launch_us": round(split_ms * 1e3, 2),
                     "kernel_source_digest": kernel_source_digest()},
        "combine_us": round(float(np.mean(r["combine_ms"])) * 1e3, 2),
        "plan": {"host_us": round(plan_us, 2), "host_c_us": round(plan_c_us, 2), "upload_us": round(upload_us, 2),
                 "per_layer_amortised_us": round((plan_c_us + upload_us) / 80, 3),
                 "map_words": int(len(step.map_host)),
                 "first_plan_and_upload_s": round(plan_s, 4), "device_us": round(plan_device_us, 2),
                 "device_map_equals_host": plan_device_exact},
    }

    # per-CU busy spread from the in-kernel timestamps (separate, instrumented run)
    timing = torch.zeros((step.W * args.head_groups, 4), dtype=torch.int64, device=dev)
    step.splitkv(q, kc, vc, bt, scale, timing=timing)
    torch.cuda.synchronize()
    result["per_cu_busy"] = per_cu_busy(timing)

    if not args.no_rated and wl.name != "tiny":
        result["xcd_rated"] = optional_section(
            "xcd_rated", lambda: rated_compare(dev, wl, step, q, caches, bt, out, args, ms_per_step * 1e3,
                                               nbytes["splitkv"]))

    if not args.no_static and wl.name != "tiny":
        max_tiles = max(-(-L // args.tile) for L in wl.kv_lens)
        plain = min(max(1, -(-step.W // wl.batch)), max_tiles)
        splits = sorted(set([plain] + [s for s in (1, 2, 4, 8, 16, 32, 64) if s <= max_tiles]))
        rows = []
        for S in splits:
            st = DecodeStep(wl.kv_lens, dev, num_q_heads=wl.hq, tile=args.tile, head_groups=args.head_groups,
                            static_splits=S)

            def s_split(i, st=st):
                k_, v_ = caches[i % copies]
                st.splitkv(q, k_, v_, bt, scale)

            rs = time_steps(s_split, lambda i, st=st: st.combine(out), args.static_steps, 2)
            tm = rs["total_ms"] / args.static_steps
            timing_s = torch.zeros((st.W * args.head_groups, 4), dtype=torch.int64, device=dev)
            st.splitkv(q, kc, vc, bt, scale, timing=timing_s)
            torch.cuda.synchronize()
            rows.append({"splits": S, "workgroups": st.W * args.head_groups, "us_per_step": round(tm * 1e3, 2),
                         "per_cu_max_over_mean": round(per_cu_busy(timing_s)["max_over_mean"], 3)})
            log(f"static S={S}: {tm * 1e3:.1f} us")
        best = min(rows, key=lambda x: x["us_per_step"])
        plain_row = next(x for x in rows if x["splits"] == plain)
        result["static_baseline"] = {
            "plain_splits": plain, "plain_us": plain_row["us_per_step"], "best_splits": best["splits"],
            "best_us": best["us_per_step"],
            "speedup_vs_plain": round(plain_row["us_per_step"] / (ms_per_step * 1e3), 3),
            "speedup_vs_best": round(best["us_per_step"] / (ms_per_step * 1e3), 3), "sweep": rows}
        # the pages' own single-operator figures for dynamic over static split-KV, on Hopper-class GPUs
        # with batches they do not specify: context beside this run's figures, not a target
        result["pages_context"] = {
            "source": "\"Hy3 Preview AI Infra 推理优化精读笔记\" §3.1 收益; "
                      "\"腾讯混元AI Infra进化：HPC-Ops推理核心算子全面升级\" §三 Attention",
            "hardware": "Hopper-class (not this machine)",
            "speedup_vs_static_mixed_lengths": [1.59, 1.76],
            "speedup_vs_static_single_long_request": 2.95,
            "this_run": {"workload": wl.name,
                         "speedup_vs_plain_static": result["static_baseline"]["speedup_vs_plain"],
                         "speedup_vs_best_static": result["static_baseline"]["speedup_vs_best"]}}

    if not args.no_static and wl.name != "tiny":
        # the LPT assignment of the fifth page (largest tile first onto the least-loaded worker)
        st = DecodeStep(wl.kv_lens, dev, num_q_heads=wl.hq, num_workers=workers, tile=args.tile,
                        head_groups=args.head_groups,
                        planner="lpt")

        def l_split(i, st=st):
            k_, v_ = caches[i % copies]
            st.splitkv(q, k_, v_, bt, scale)

        rl = time_steps(l_split, lambda i, st=st: st.combine(out), args.static_steps, 2)
        timing_l = torch.zeros((st.W * args.head_groups, 4), dtype=torch.int64, device=dev)
        st.splitkv(q, kc, vc, bt, scale, timing=timing_l)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            lb.attn_plan_lpt(wl.kv_lens, workers, args.tile)
        lpt_host_us = (time.perf_counter() - t0) / 5 * 1e6
        result["lpt_baseline"] = {
            "segments": st.S, "us_per_step": round(rl["total_ms"] / args.static_steps * 1e3, 2),
            "splitkv_us": round(float(np.mean(rl["split_ms"])) * 1e3, 2),
            "combine_us": round(float(np.mean(rl["combine_ms"])) * 1e3, 2),
            "per_cu_max_over_mean": round(per_cu_busy(timing_l)["max_over_mean"], 3),
            "host_plan_us": round(lpt_host_us, 1),
            "dynamic_speedup": round(rl["total_ms"] / args.static_steps / ms_per_step, 3)}
        log(f"lpt map: S={st.S}, step {result['lpt_baseline']['us_per_step']} us")
        del st

    if not args.no_static and wl.name != "tiny":
        # the cost-weighted contiguous fill (tile cost in tokens plus a per-request split cost) at a
        # few tile sizes and split costs
        rows = []
        for planner, tile_w, sc in (("greedy", 128, 0), ("greedy", 64, 0), ("weighted", 512, 0), ("weighted", 512, 128),
                                    ("weighted", 128, 0), ("weighted", 128, 128), ("weighted", 64, 256)):
            st = DecodeStep(wl.kv_lens, dev, num_q_heads=wl.hq, num_workers=workers, tile=tile_w,
                            head_groups=args.head_groups,
                            planner=planner, split_cost=sc)

            def w_split(i, st=st):
                k_, v_ = caches[i % copies]
                st.splitkv(q, k_, v_, bt, scale)

            rw = time_steps(w_split, lambda i, st=st: st.combine(out), args.static_steps, 2)
            timing_w = torch.zeros((st.W * args.head_groups, 4), dtype=torch.int64, device=dev)
            st.splitkv(q, kc, vc, bt, scale, timing=timing_w)
            torch.cuda.synchronize()
            us = rw["total_ms"] / args.static_steps * 1e3
            rows.append({"planner": planner, "tile": tile_w, "split_cost": sc, "segments": st.S,
                         "us_per_step": round(us, 2),
                         "splitkv_us": round(float(np.mean(rw["split_ms"])) * 1e3, 2),
                         "combine_us": round(float(np.mean(rw["combine_ms"])) * 1e3, 2),
                         "per_cu_max_over_mean": round(per_cu_busy(timing_w)["max_over_mean"], 3),
                         "greedy_speedup": round(us / (ms_per_step * 1e3), 3)})
            log(f"{planner} map tile={tile_w} split_cost={sc}: S={st.S}, step {us:.1f} us")
            del st
        result["weighted_baseline"] = {
            "what": "cost-weighted contiguous fill: tile cost = KV tokens + split_cost on a request's first "
                    "tile, tile to the worker whose equal cost share holds its midpoint; beside it the greedy "
                    "fill at smaller tiles; greedy_speedup = this step / the 512-token greedy-fill step",
            "sweep": rows}

    if not args.no_claim and wl.hkv == args.head_groups:
        result["claimed"] = claim_sweep(dev, wl, q, caches, bt, out, args, ms_per_step * 1e3)

    if not args.no_probe:
        # the device's streaming-read ceiling, measured on the same run (the KV cache itself)
        sink = torch.zeros(8192 * 256, dtype=torch.int32, device=dev)
        best = None
        for blocks in (1024, 2048, 4096):
            for _ in range(2):
                lb.attn_probe_stream_read(kc, blocks, sink)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                lb.attn_probe_stream_read(kc, blocks, sink)
            e1.record()
            torch.cuda.synchronize()
            gbs = kc.numel() * 2 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
            best = gbs if best is None else max(best, gbs)
        result["stream_read_ceiling"] = {"GB/s": round(best, 1), "buffer_GB": round(kc.numel() * 2 / 1e9, 2),
                                         "splitkv_frac_of_ceiling": round(achieved / best, 4)}
        rated = result.get("xcd_rated")
        if rated and "error" not in rated:
            # the same read with each XCD's share in proportion to the rates calibrated above: the
            # ceiling for work shared out by XCD rate (equal shares leave the faster XCDs idle at the end)
            best_r = None
            for blocks in (1024, 2048, 4096):
                for _ in range(2):
                    lb.attn_probe_stream_read_rated(kc, blocks, rated["xcd_rates"], sink)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    lb.attn_probe_stream_read_rated(kc, blocks, rated["xcd_rates"], sink)
                e1.record()
                torch.cuda.synchronize()
                gbs = kc.numel() * 2 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
                best_r = gbs if best_r is None else max(best_r, gbs)
            row = next(x for x in rated["sweep"] if x["map"] == "list-major, calibrated rates")
            rated_gbs = nbytes["splitkv"] / (row["splitkv_us"] * 1e-6) / 1e9
            result["stream_read_ceiling"].update({
                "xcd_rated_GB/s": round(best_r, 1),
                "splitkv_frac_of_xcd_rated_ceiling": round(achieved / best_r, 4),
                "rated_map_splitkv_frac_of_xcd_rated_ceiling": round(rated_gbs / best_r, 4)})
            log(f"streaming-read ceiling {best:.0f} GB/s, with per-XCD shares {best_r:.0f} GB/s")

    if not args.no_fp8:
        result["fp8_kv"] = bench_fp8(dev, wl, args, ms_per_step * 1e3)

    if not args.no_mtp and wl.name != "tiny":
        result["mtp"] = bench_mtp(dev, wl.name, args, ms_per_step * 1e3)

    if not args.no_store and wl.name != "tiny":
        result["store_kv"] = bench_store_kv(dev, wl, args)

    legs = [x for x in args.legs.split(",") if x and x != wl.name]
    if legs:
        result["legs"] = {name: bench_decode_leg(dev, name, args) for name in legs}

    if not args.no_prefill:
        result["prefill"] = bench_prefill(dev, *prefill_args)

    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a CPU sample")
        result["cpu_baseline"] = cpu_oracle_baseline(wl, args.cpu_seconds, scale, workers, args.tile)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
