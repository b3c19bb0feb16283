"""C ABI on the CPU: the library loads, exports every declared symbol, and its host planner
reproduces the oracle's work map bit for bit (no GPU calls here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import workloads as WL
from oracle.plan import ref_plan, ref_plan_prefill, ref_plan_static

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for hdr in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if hdr.endswith(".h"):
            src = open(os.path.join(ROOT, "include", hdr)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(attn_[a-z_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    import load_balanced_split_attn_amd as lb
    return lb


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert len(names) >= 8
    handle = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n


def test_status_strings(L):
    assert L.attn_status_string(0) == "ok"
    assert L.attn_status_string(-2) == "map buffer too small"


def _random_batches(n, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        B = int(rng.integers(0, 20))
        tile = int(rng.choice([1, 32, 64, 512]))
        hi = int(rng.choice([1, 3, 40])) * tile
        lens = [int(x) for x in rng.integers(0, hi + 2, size=B)]
        W = int(rng.integers(1, 300))
        yield lens, W, tile


def test_plan_bit_exact_random(L):
    for lens, W, tile in _random_batches(3000, 1):
        got = L.attn_plan(lens, W, tile)
        exp = ref_plan(lens, W, tile)
        assert got.dtype == np.int32 and np.array_equal(got, exp), (lens, W, tile)


def test_plan_static_bit_exact_random(L):
    for lens, W, tile in _random_batches(2000, 2):
        S = 1 + W % 17
        assert np.array_equal(L.attn_plan_static(lens, S, tile), ref_plan_static(lens, S, tile)), (lens, S, tile)


def test_plan_prefill_bit_exact_random(L):
    rng = np.random.default_rng(3)
    for _ in range(1500):
        B = int(rng.integers(0, 8))
        q_lens = [int(x) for x in rng.integers(0, 600, size=B)]
        kv_lens = [q + int(rng.integers(0, 5000)) for q in q_lens]
        W = int(rng.integers(1, 200))
        q_tile = int(rng.choice([16, 128]))
        kv_tile = int(rng.choice([64, 512]))
        causal = bool(rng.integers(0, 2))
        got = L.attn_plan_prefill(q_lens, kv_lens, W, q_tile, kv_tile, causal)
        exp = ref_plan_prefill(q_lens, kv_lens, W, q_tile, kv_tile, causal)
        assert np.array_equal(got, exp), (q_lens, kv_lens, W, q_tile, kv_tile, causal)


@pytest.mark.parametrize("name", ["tiny", "uniform", "mixed", "long_tail", "control"])
@pytest.mark.parametrize("W", [4, 256, 384, 512, 1024])
def test_plan_bit_exact_workloads(L, name, W):
    wl = WL.BY_NAME[name]()
    assert np.array_equal(L.attn_plan(wl.kv_lens, W, 512), ref_plan(wl.kv_lens, W, 512))
    for S in (1, 2, 7, 13, 64):
        assert np.array_equal(L.attn_plan_static(wl.kv_lens, S, 512), ref_plan_static(wl.kv_lens, S, 512))


@pytest.mark.parametrize("W", [64, 256, 1024])
def test_plan_prefill_bit_exact_workload(L, W):
    wl = WL.prefill()
    got = L.attn_plan_prefill(wl.q_lens, wl.kv_lens, W, 128, 512, True)
    assert np.array_equal(got, ref_plan_prefill(wl.q_lens, wl.kv_lens, W, 128, 512, True))


def test_map_words_bound(L):
    for lens, W, tile in _random_batches(500, 4):
        words = L.attn_plan(lens, W, tile)
        T = int(words[5])
        assert len(words) <= L.attn_map_words(len(lens), W, T)
    assert L.lib().attn_map_words(-1, 3, 5) == -1


def test_errors_and_capacity(L):
    lib = L.lib()
    i32 = ctypes.c_int32
    lens = (i32 * 3)(1024, 5120, 2048)
    buf = (i32 * 64)()
    need = i32(0)
    assert lib.attn_plan(lens, 3, 4, 512, buf, 10, ctypes.byref(need)) == -2
    assert need.value == 8 + 5 + 4 + 6 + 4 * 5
    assert lib.attn_plan(lens, 3, 4, 512, buf, need.value, ctypes.byref(need)) == 0
    assert list(buf)[:need.value] == ref_plan([1024, 5120, 2048], 4, 512).tolist()
    bad = (i32 * 2)(5, -1)
    assert lib.attn_plan(bad, 2, 4, 512, buf, 64, None) == -1
    assert lib.attn_plan(lens, 3, 0, 512, buf, 64, None) == -1
    assert lib.attn_plan(lens, 3, 4, 0, buf, 64, None) == -1
    assert lib.attn_plan(lens, -1, 4, 512, buf, 64, None) == -1
    assert lib.attn_plan(None, 3, 4, 512, buf, 64, None) == -1
    assert lib.attn_plan_static(lens, 3, 0, 512, buf, 64, None) == -1
    ql = (i32 * 1)(10)
    kl = (i32 * 1)(5)
    assert lib.attn_plan_prefill(ql, kl, 1, 4, 128, 512, 1, buf, 64, None) == -1
    # kernels reject bad shapes before touching the device
    assert lib.attn_splitkv(None, None, None, None, 0, 1, None, None, 4, 0, 8, 1, 64, 8, 128, 64, 1.0,
                            None, None, None, None, None) == -1
    dummy = ctypes.c_void_p(16)
    assert lib.attn_splitkv(dummy, dummy, dummy, dummy, 1, 1, dummy, dummy, 4, 0, 8, 1, 64, 8, 96, 64, 1.0,
                            None, None, None, None, None) == -3
    # the 8-bit cache entry point also needs both scale arrays
    assert lib.attn_splitkv_fp8(dummy, dummy, dummy, None, dummy, dummy, 1, 1, dummy, dummy, 4, 0, 8, 1, 64, 8,
                                128, 64, 1.0, None, None, None, None, None) == -1
    assert lib.attn_splitkv_fp8(dummy, dummy, dummy, dummy, dummy, dummy, 1, 1, dummy, dummy, 4, 0, 8, 1, 64, 8,
                                96, 64, 1.0, None, None, None, None, None) == -3
    # multi-token decode: q_lens/q_start required, kv_dtype and scales must agree, at most 4 rows
    def mtp(kv_dtype, ks, vs, q_lens, rows, head_dim=128):
        return lib.attn_splitkv_mtp(dummy, dummy, dummy, kv_dtype, ks, vs, dummy, 1, 1, q_lens, q_lens, dummy,
                                    dummy, 4, 0, 8, 1, 64, 8, head_dim, 64, rows, 1.0, None, None, None, None)
    assert mtp(0, None, None, None, 2) == -1
    assert mtp(5, None, None, dummy, 2) == -1
    assert mtp(0, dummy, dummy, dummy, 2) == -1
    assert mtp(1, None, None, dummy, 2) == -1
    assert mtp(0, None, None, dummy, 5) == -3
    assert mtp(1, dummy, dummy, dummy, 0) == -1
    assert mtp(0, None, None, dummy, 2, head_dim=64) == -3
    # device planner: host-side argument checks (no launch)
    assert lib.attn_plan_device(dummy, -1, 4, 512, dummy, 100, None) == -1
    assert lib.attn_plan_device(dummy, 3, 0, 512, dummy, 100, None) == -1
    assert lib.attn_plan_device(dummy, 3, 4, 0, dummy, 100, None) == -1
    assert lib.attn_plan_device(dummy, 3, 4, 512, None, 100, None) == -1
    assert lib.attn_plan_device(None, 3, 4, 512, dummy, 100, None) == -1
    assert lib.attn_plan_device(dummy, 3, 4, 512, dummy, 8 + 5 + 4 + 6 - 1, None) == -2
    # producer step: argument checks before any launch
    def store(**kw):
        a = dict(q=dummy, k=dummy, v=dummy, qw=None, kw=None, eps=1e-6, pos=dummy, theta=0.0, had=0, qo=dummy,
                 kc=dummy, vc=dummy, dt=0, ks=None, vs=None, bt=dummy, bts=1, np_=1, B=1, Hq=64, Hkv=8, D=128,
                 page=64)
        a.update(kw)
        return lib.attn_store_kv(a["q"], a["k"], a["v"], a["qw"], a["kw"], a["eps"], a["pos"], a["theta"], a["had"],
                                 a["qo"], a["kc"], a["vc"], a["dt"], a["ks"], a["vs"], a["bt"], a["bts"], a["np_"],
                                 a["B"], a["Hq"], a["Hkv"], a["D"], a["page"], None)
    assert store(q=None) == -1
    assert store(had=2) == -1
    assert store(eps=-1.0) == -1
    assert store(theta=float("nan")) == -1
    assert store(dt=1) == -1                 # E4M3 without scales
    assert store(dt=3, ks=dummy, vs=dummy) == -1
    assert store(D=64) == -3
    assert store(page=48) == -3
    assert store(B=0, q=None) == 0           # nothing to do
    out = ctypes.c_int32(0)
    assert lib.attn_query_workers(0, 8, 7, ctypes.byref(out)) == -1
    assert lib.attn_query_workers(0, 3, 0, ctypes.byref(out)) == -1
    assert lib.attn_combine(None, None, None, dummy, 1, 1, None, None, 64, 128, None, 0, 0, None) == -1
    assert lib.attn_combine(dummy, dummy, dummy, dummy, 1, 1, None, None, 64, 128, dummy, 0, -1, None) == -1
    # measurement probes: argument checks before any launch
    assert lib.attn_probe_stream_read(None, 16, 1, dummy, None) == -1
    assert lib.attn_probe_stream_read(dummy, 15, 1, dummy, None) == -1
    assert lib.attn_probe_stream_read(dummy, 16, 0, dummy, None) == -1
    rates8 = (ctypes.c_int32 * 8)(1, 1, 1, 1, 1, 1, 1, 1)
    zeros8 = (ctypes.c_int32 * 8)()
    assert lib.attn_probe_stream_read_rated(dummy, 16, 12, rates8, dummy, None) == -1     # not a multiple of 8
    assert lib.attn_probe_stream_read_rated(dummy, 16, 0, rates8, dummy, None) == -1
    assert lib.attn_probe_stream_read_rated(dummy, 16, 8, zeros8, dummy, None) == -1
    assert lib.attn_probe_stream_read_rated(dummy, 16, 8, None, dummy, None) == -1
    assert lib.attn_probe_stream_read_rated(None, 16, 8, rates8, dummy, None) == -1
    assert lib.attn_probe_mfma_rate(0, 1, dummy, None) == -1
    assert lib.attn_probe_mfma_rate(1, 0, dummy, None) == -1
    assert lib.attn_probe_mfma_rate(1, 1, None, None) == -1
    assert lib.attn_probe_mfma_rate(1, 1, ctypes.c_void_p(18), None) == -1


def test_weighted_plan_bit_exact():
    """attn_plan_weighted (C++) reproduces the oracle's cost-weighted map word for word: random
    batches with empty requests and partial tiles, several split costs, and the bench workloads at
    the tile sizes and split costs the bench compares."""
    import load_balanced_split_attn_amd as lb
    from oracle.plan import ref_plan_weighted
    rng = np.random.default_rng(23)
    for _ in range(600):
        B = int(rng.integers(0, 14))
        W = int(rng.integers(1, 24))
        tile = int(rng.choice([16, 64, 128, 512]))
        sc = int(rng.choice([0, 1, 64, 256, 5000]))
        lens = [int(x) if rng.random() > 0.2 else 0 for x in rng.integers(1, 5000, size=B)]
        got = lb.attn_plan_weighted(lens, W, tile, sc)
        assert np.array_equal(got, ref_plan_weighted(lens, W, tile, sc)), (lens, W, tile, sc)
    import workloads as WL
    for name in ("tiny", "uniform", "mixed", "long_tail"):
        wl = WL.BY_NAME[name]()
        W = wl.workers or 128
        for tile, sc in ((512, 0), (512, 128), (128, 128), (64, 256)):
            assert np.array_equal(lb.attn_plan_weighted(wl.kv_lens, W, tile, sc),
                                  ref_plan_weighted(wl.kv_lens, W, tile, sc)), (name, tile, sc)
    # lengths at the int32 limit: the cost products need more than 64 bits of headroom
    big = [2**31 - 1, 2**31 - 1, 5]
    assert np.array_equal(lb.attn_plan_weighted(big, 7, 2**20, 2**30), ref_plan_weighted(big, 7, 2**20, 2**30))


def test_weighted_plan_errors():
    import load_balanced_split_attn_amd as lb
    for args in (([10], 2, 64, -1), ([10], 0, 64, 0), ([10], 2, 0, 0), ([-1], 2, 64, 0)):
        with pytest.raises(lb.LbsaError):
            lb.attn_plan_weighted(*args)


def test_rated_plan_bit_exact():
    """attn_plan_rated (C++) reproduces the oracle's rate-proportional map word for word: random
    batches with empty requests and partial tiles, random rates with zeros (leading, trailing and
    inside), split costs, the bench workloads at per-XCD rates like the device's, and lengths and
    rates at their limits."""
    import load_balanced_split_attn_amd as lb
    from oracle.plan import RATE_MAX, ref_plan_rated
    rng = np.random.default_rng(29)
    for _ in range(600):
        B = int(rng.integers(0, 14))
        W = int(rng.integers(1, 24))
        tile = int(rng.choice([16, 64, 128, 512]))
        sc = int(rng.choice([0, 1, 64, 256, 5000]))
        lens = [int(x) if rng.random() > 0.2 else 0 for x in rng.integers(1, 5000, size=B)]
        hi = int(rng.choice([2, 100, RATE_MAX]))
        rates = [int(x) if rng.random() > 0.25 else 0 for x in rng.integers(1, hi + 1, size=W)]
        if sum(rates) == 0:
            rates[-1] = 1
        got = lb.attn_plan_rated(lens, W, rates, tile, sc)
        assert np.array_equal(got, ref_plan_rated(lens, W, tile, sc, rates)), (lens, W, tile, sc, rates)
    import workloads as WL
    xcd = [65536, 61440, 65000, 61900, 64800, 62000, 65536, 61000]
    for name in ("tiny", "uniform", "mixed", "long_tail", "mixed_tp8"):
        wl = WL.BY_NAME[name]()
        W = wl.workers or 128
        rates = [xcd[w % 8] for w in range(W)]
        for tile, sc in ((512, 0), (128, 0), (64, 256)):
            assert np.array_equal(lb.attn_plan_rated(wl.kv_lens, W, rates, tile, sc),
                                  ref_plan_rated(wl.kv_lens, W, tile, sc, rates)), (name, tile, sc)
    big = [2**31 - 1, 2**31 - 1, 5]
    rates = [RATE_MAX, 1, 0, RATE_MAX - 1, 7, 0, RATE_MAX]
    assert np.array_equal(lb.attn_plan_rated(big, 7, rates, 2**20, 2**30),
                          ref_plan_rated(big, 7, 2**20, 2**30, rates))


def test_rated_plan_errors():
    import load_balanced_split_attn_amd as lb
    for args in (([10], 2, [1, 1], 64, -1), ([10], 2, [0, 0], 64, 0), ([10], 2, [1, -1], 64, 0),
                 ([10], 2, [1, lb.RATE_MAX + 1], 64, 0), ([10], 2, [1, 1], 0, 0), ([-1], 2, [1, 1], 64, 0)):
        with pytest.raises(lb.LbsaError):
            lb.attn_plan_rated(*args)
    with pytest.raises(ValueError):
        lb.attn_plan_rated([10], 2, [1, 1, 1])
    L = lb.lib()
    i32 = ctypes.c_int32
    buf = (i32 * 64)()
    assert L.attn_plan_rated((i32 * 1)(10), 1, 2, 64, 0, None, buf, 64, None) == -1


def test_xcd_rates_from_timing():
    """Per-XCD rates from synthetic timestamp records: XCD x's workgroups take d_x per token, so its
    rate is 1 / d_x, for a version-1 map with eight head groups (workgroup b on list b // 8, every
    XCD one head group of every list) and for a version-3 map (list b mod W, lists on XCD w mod 8)."""
    import torch

    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.decode import xcd_rates_from_timing
    lens = [1000, 3000, 512, 7000, 0, 2222, 4096, 100, 9000, 333]
    speed = np.array([1.0, 0.95, 1.0, 0.93, 0.99, 0.94, 1.0, 0.96])
    for words in (lb.attn_plan(lens, 16, 128), lb.attn_plan_rated(lens, 16, [3] * 16, 128)):
        hdr = lb.map_header(words)
        W = hdr["W"]
        wptr = words[8:8 + W + 1]
        segs = words[8 + (W + 1) + (hdr["U"] + 1) + 2 * hdr["U"]:].reshape(-1, 4)
        tokens = [int((segs[wptr[w]:wptr[w + 1], 3] - segs[wptr[w]:wptr[w + 1], 2]).sum()) for w in range(W)]
        rows = []
        for rep in range(2):
            for b in range(W * 8):
                w = b % W if hdr["version"] == 3 else b // 8
                x = b % 8
                start = 1000 * rep + b
                rows.append([start, start + int(round(tokens[w] / speed[x] * 1000)) + 1, 0, x])
        got = xcd_rates_from_timing(torch.tensor(rows, dtype=torch.int64), words, 8)
        want = np.round(65536 * speed / speed.max())
        assert np.max(np.abs(np.array(got) - want)) <= 40, (got, want)


def test_xcd_token_balance():
    """Per-XCD token totals under list-major placement (list w on XCD w mod 8), against sums taken
    directly from the oracle's segments: equal on the uniform and mixed batches (whole tiles, budgets
    that differ by one tile spread over the XCDs alike), 1.9% apart on the long-tail batch."""
    import workloads as WL
    from load_balanced_split_attn_amd.decode import LIST_MAJOR_BALANCE, list_tokens, xcd_token_balance
    from oracle.plan import parse_map, ref_plan
    for name, want in (("uniform", 1.0), ("mixed", 1.0), ("long_tail", 1.0190)):
        words = ref_plan(WL.BY_NAME[name]().kv_lens, 128, 512)
        mp = parse_map(words)
        direct = np.array([sum(e - a for _, _, a, e in mp.worker_segments(w).tolist()) for w in range(mp.W)])
        assert np.array_equal(list_tokens(words), direct)
        per_xcd = np.array([direct[x::8].sum() for x in range(8)])
        assert xcd_token_balance(words) == pytest.approx(per_xcd.max() / per_xcd.mean())
        assert xcd_token_balance(words) == pytest.approx(want, abs=5e-4)
    assert xcd_token_balance(ref_plan(WL.BY_NAME["long_tail"]().kv_lens, 128, 512)) > LIST_MAJOR_BALANCE
    assert xcd_token_balance(ref_plan([0, 0], 16, 512)) == 1.0


def test_lpt_plan_bit_exact():
    """attn_plan_lpt (C++) reproduces the oracle's version-2 LPT map word for word."""
    import load_balanced_split_attn_amd as lb
    from oracle.plan import ref_plan_lpt
    rng = np.random.default_rng(21)
    for _ in range(400):
        B = int(rng.integers(0, 12))
        W = int(rng.integers(1, 20))
        tile = int(rng.choice([16, 64, 512]))
        lens = [int(x) for x in rng.integers(0, 4000, size=B)]
        assert np.array_equal(lb.attn_plan_lpt(lens, W, tile), ref_plan_lpt(lens, W, tile)), (lens, W, tile)
    import workloads as WL
    for name in ("tiny", "uniform", "mixed", "long_tail"):
        wl = WL.BY_NAME[name]()
        W = wl.workers or 128
        assert np.array_equal(lb.attn_plan_lpt(wl.kv_lens, W, 512), ref_plan_lpt(wl.kv_lens, W, 512)), name


def test_binding_refuses_undersized_partials(L):
    """The binding checks every partial buffer's size (part_l included) before anything reaches the
    library: an undersized one is a ValueError, never a launch writing past its end.  CPU tensors
    suffice, since the sizes are checked before the device."""
    import torch
    S, Hq, D = 3, 64, 128
    q = torch.zeros((2, Hq, D), dtype=torch.bfloat16)
    other = torch.zeros(1, dtype=torch.int32)
    for rows, call in ((1, lambda m, l, o: L.attn_splitkv(q, q, q, other, other, other, 4, S, 8, 0.1, m, l, o)),
                       (1, lambda m, l, o: L.attn_splitkv_fp8(q, q, q, other, other, other, other, other, 4, S, 8,
                                                              0.1, m, l, o)),
                       (4, lambda m, l, o: L.attn_splitkv_mtp(q, q, q, other, other, other, other, other, 4, S, 8,
                                                              4, 0.1, m, l, o)),
                       (128, lambda m, l, o: L.attn_splitkv_prefill(q, q, q, other, other, other, other, other, 4,
                                                                    S, 0.1, m, l, o, q_tile=128))):
        n = S * rows * Hq
        full = (torch.zeros(n), torch.zeros(n), torch.zeros(n * D))
        for i, name in enumerate(("part_m", "part_l", "part_o")):
            bufs = list(full)
            bufs[i] = torch.zeros(bufs[i].numel() - 1)
            with pytest.raises(ValueError, match=name):
                call(*bufs)
