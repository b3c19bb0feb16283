"""Pins for the oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes the oracle function(s) under test as arguments and
raises AssertionError when they disagree with what the pages or the mathematics
fix.  ``test_oracle_*.py`` runs every pin on the real oracle; ``test_oracle_mutations.py``
runs them on copies of the oracle with a planted mistake and requires that some
pin fails for each.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------------------------------------
# Brute force: a pure-Python softmax with exact summation (math.fsum), written from the definition.

def brute_attention(q, k, v, scale, q_len, kv_len, causal, first_row=0):
    """q: nested [R][Hq][D] floats, k/v: [L][Hkv][D].  Returns [R][Hq][D]."""
    R = len(q)
    Hq = len(q[0])
    D = len(q[0][0])
    Hkv = len(k[0]) if kv_len else 1
    per = Hq // Hkv
    out = []
    for j in range(R):
        row = []
        last = (kv_len - q_len + first_row + j) if causal else kv_len - 1
        for h in range(Hq):
            g = h // per
            keys = [t for t in range(kv_len) if t <= last]
            if not keys:
                row.append([0.0] * D)
                continue
            s = [scale * math.fsum(q[j][h][d] * k[t][g][d] for d in range(D)) for t in keys]
            mx = max(s)
            p = [math.exp(x - mx) for x in s]
            den = math.fsum(p)
            row.append([math.fsum(p[i] * v[t][g][d] for i, t in enumerate(keys)) / den for d in range(D)])
        out.append(row)
    return out


def _bf16_np(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(torch.bfloat16).to(torch.float64).numpy()


def pin_bruteforce_decode(ref_attention, trials=12):
    """Decode rows (one query at position L-1) against the fsum brute force, Hq=4, Hkv=2."""
    for t in range(trials):
        L = 1 + (t * 5) % 12
        D = 1 + t % 4
        q = _bf16_np((1, 4, D), 10 + t)
        k = _bf16_np((L, 2, D), 20 + t)
        v = _bf16_np((L, 2, D), 30 + t)
        scale = 1.0 / math.sqrt(D) * (1.0 + 0.37 * t)
        got = ref_attention(q, k, v, scale, causal=True)
        exp = np.array(brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, 1, L, True))
        assert np.allclose(got, exp, rtol=1e-13, atol=1e-13), f"decode trial {t}"


def pin_bruteforce_prefill(ref_attention, trials=8):
    """Causal chunk rows after a cached prefix, and the non-causal case, against brute force."""
    for t in range(trials):
        prefix = t % 5
        R = 1 + (t * 3) % 6
        L = prefix + R
        D = 2 + t % 3
        q = _bf16_np((R, 4, D), 40 + t)
        k = _bf16_np((L, 2, D), 50 + t)
        v = _bf16_np((L, 2, D), 60 + t)
        scale = 0.5 + 0.1 * t
        for causal in (True, False):
            got = ref_attention(q, k, v, scale, causal=causal)
            exp = np.array(brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, R, L, causal))
            assert np.allclose(got, exp, rtol=1e-13, atol=1e-13), f"prefill trial {t} causal={causal}"


def pin_closed_forms(ref_attention):
    """Closed forms that any exact softmax attention must satisfy."""
    rng = np.random.default_rng(7)
    L, Hq, Hkv, D = 37, 8, 2, 16
    q = rng.standard_normal((1, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    # all value rows equal c -> output c
    c = rng.standard_normal(D)
    v = np.broadcast_to(c, (L, Hkv, D)).copy()
    out = ref_attention(q, k, v, 0.3)
    assert np.allclose(out, np.broadcast_to(c, out.shape), atol=1e-12)
    # q = 0 -> uniform weights -> mean of the value rows
    v = rng.standard_normal((L, Hkv, D))
    out = ref_attention(np.zeros_like(q), k, v, 0.3)
    for h in range(Hq):
        assert np.allclose(out[0, h], v[:, h // (Hq // Hkv)].mean(axis=0), atol=1e-12)
    # one key -> its value row
    out = ref_attention(q, k[:1], v[:1], 0.3)
    for h in range(Hq):
        assert np.allclose(out[0, h], v[0, h // (Hq // Hkv)], atol=1e-12)
    # a single dominant key: softmax puts (almost) all weight on it
    k2 = k.copy()
    k2[11] = 40.0 * q[0, 0] / np.linalg.norm(q[0, 0])          # head 0 aligns with key 11
    out = ref_attention(q, k2, v, 1.0)
    assert np.allclose(out[0, 0], v[11, 0], atol=1e-9)
    # heads of one group with equal queries give equal outputs; heads of another group differ
    q3 = np.repeat(q[:, :1], Hq, axis=1)
    out = ref_attention(q3, k, v, 0.3)
    per = Hq // Hkv
    for h in range(Hq):
        assert np.allclose(out[0, h], out[0, (h // per) * per], atol=1e-14)
    assert not np.allclose(out[0, 0], out[0, per])


def pin_gqa_head_map(ref_attention):
    """Changing KV head g changes exactly the query heads g*per .. g*per+per-1."""
    rng = np.random.default_rng(8)
    L, Hq, Hkv, D = 9, 8, 4, 8
    q = rng.standard_normal((1, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    base = ref_attention(q, k, v, 0.5)
    per = Hq // Hkv
    for g in range(Hkv):
        v2 = v.copy()
        v2[:, g] += 1.0
        out = ref_attention(q, k, v2, 0.5)
        changed = [h for h in range(Hq) if not np.allclose(out[0, h], base[0, h])]
        assert changed == list(range(g * per, (g + 1) * per)), (g, changed)


def pin_library_sdpa(ref_attention):
    """With no cached prefix the causal chunk is textbook causal attention: compare against
    torch's scaled_dot_product_attention in float64 (GQA expanded by repeating KV heads)."""
    g = torch.Generator().manual_seed(3)
    for (R, Hq, Hkv, D, prefix) in [(13, 8, 2, 16, 0), (7, 4, 4, 8, 0), (5, 8, 1, 32, 0)]:
        q = torch.randn(R, Hq, D, generator=g, dtype=torch.float64)
        k = torch.randn(R + prefix, Hkv, D, generator=g, dtype=torch.float64)
        v = torch.randn(R + prefix, Hkv, D, generator=g, dtype=torch.float64)
        per = Hq // Hkv
        kk = k.repeat_interleave(per, dim=1).permute(1, 0, 2)
        vv = v.repeat_interleave(per, dim=1).permute(1, 0, 2)
        exp = torch.nn.functional.scaled_dot_product_attention(
            q.permute(1, 0, 2), kk, vv, is_causal=True, scale=0.25).permute(1, 0, 2).numpy()
        got = ref_attention(q.numpy(), k.numpy(), v.numpy(), 0.25, causal=True)
        assert np.allclose(got, exp, rtol=1e-12, atol=1e-12)
        exp_nc = torch.nn.functional.scaled_dot_product_attention(
            q.permute(1, 0, 2), kk, vv, is_causal=False, scale=0.25).permute(1, 0, 2).numpy()
        got_nc = ref_attention(q.numpy(), k.numpy(), v.numpy(), 0.25, causal=False)
        assert np.allclose(got_nc, exp_nc, rtol=1e-12, atol=1e-12)


def pin_combine_invariance(ref_attention, ref_partial, ref_combine, trials=30):
    """Any partition of the KV range, merged by combine, equals the unsplit result (fp64)."""
    rng = np.random.default_rng(11)
    for t in range(trials):
        L = int(rng.integers(1, 200))
        R = int(rng.integers(1, 5))
        causal = bool(t % 2)
        Lctx = L + (R if causal else 0)
        q = rng.standard_normal((R, 4, 8)) * 2.0
        k = rng.standard_normal((Lctx, 2, 8))
        v = rng.standard_normal((Lctx, 2, 8))
        cuts = sorted(set([0, Lctx] + rng.integers(0, Lctx + 1, size=int(rng.integers(0, 8))).tolist()))
        # include a one-token piece and an empty piece
        parts = [ref_partial(q, k, v, 0.4, a, e, causal) for a, e in zip(cuts[:-1], cuts[1:])]
        parts.append(ref_partial(q, k, v, 0.4, Lctx, Lctx, causal))
        got = ref_combine(parts)
        exp = ref_attention(q, k, v, 0.4, causal=causal)
        assert np.allclose(got, exp, rtol=1e-13, atol=1e-13), f"trial {t}"


def pin_partial_definition(ref_partial):
    """(m, l, o) of a piece against the fsum brute force of its own definition."""
    rng = np.random.default_rng(12)
    L, D = 10, 3
    q = rng.standard_normal((1, 2, D))
    k = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    a, e = 3, 8
    m, l, o = ref_partial(q, k, v, 0.7, a, e, True)
    for h in range(2):
        s = [0.7 * math.fsum(q[0, h, d] * k[t, 0, d] for d in range(D)) for t in range(a, e)]
        mx = max(s)
        assert abs(m[0, h] - mx) < 1e-14
        assert abs(l[0, h] - math.fsum(math.exp(x - mx) for x in s)) < 1e-13
        for d in range(D):
            ref = math.fsum(math.exp(s[i] - mx) * v[a + i, 0, d] for i in range(e - a))
            assert abs(o[0, h, d] - ref) < 1e-13
    # a piece with no visible key
    m, l, o = ref_partial(q, k, v, 0.7, 5, 5, True)
    assert np.all(np.isneginf(m)) and np.all(l == 0) and np.all(o == 0)


# ------------------------------------------------------------------------------------------------
# Planner pins

def load_worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def pin_worked_example(ref_plan, parse_map):
    """The pages' worked example: tiles 2/10/4, 4 tiles per worker, the long request spans workers."""
    ex = load_worked_example()
    mp = parse_map(ref_plan(ex["seq_lens"], ex["num_workers"], ex["tile"]))
    assert mp.T == sum(ex["tiles_per_request"])
    per_req = [0] * len(ex["seq_lens"])
    per_worker = []
    for w in range(mp.W):
        n = 0
        for b, _, a, e in mp.worker_segments(w):
            t = -(-(int(e) - int(a)) // ex["tile"])
            per_req[b] += t
            n += t
        per_worker.append(n)
    assert per_req == ex["tiles_per_request"]
    assert per_worker == ex["tiles_per_worker"]
    workers_of = {}
    for w in range(mp.W):
        for b, *_ in mp.worker_segments(w):
            workers_of.setdefault(int(b), set()).add(w)
    assert ex["long_request_spans_workers"] == (len(workers_of[1]) > 1)


def _worker_of_stream_index(j, T, W):
    """Closed form of the contiguous fill: the first rem workers own base+1 consecutive indices."""
    base, rem = divmod(T, W)
    if j < rem * (base + 1):
        return j // (base + 1)
    return rem + (j - rem * (base + 1)) // base


def pin_fill_closed_form(ref_plan, parse_map, trials=400, seed=5):
    """Rebuild every segment from the per-tile closed form above and compare with the map."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        B = int(rng.integers(0, 9))
        tile = int(rng.choice([1, 3, 64, 512]))
        lens = [int(x) for x in rng.integers(0, 6 * tile + 2, size=B)]
        W = int(rng.integers(1, 12))
        mp = parse_map(ref_plan(lens, W, tile))
        stream = [(b, t) for b, L in enumerate(lens) for t in range(-(-L // tile))]
        T = len(stream)
        assert mp.T == T and mp.W == W and mp.U == B and mp.B == B
        expect = [[] for _ in range(W)]
        for j, (b, t) in enumerate(stream):
            w = _worker_of_stream_index(j, T, W)
            lst = expect[w]
            if lst and lst[-1][0] == b and lst[-1][3] == t * tile:
                lst[-1][3] = min(lens[b], (t + 1) * tile)
            else:
                lst.append([b, 0, t * tile, min(lens[b], (t + 1) * tile)])
        for w in range(W):
            assert mp.worker_segments(w).tolist() == expect[w], (lens, W, tile, w)


def pin_budget_rule(ref_plan, parse_map, trials=300, seed=6):
    """[P2]'s budgets: base = T // W for everyone, one extra for the first T % W workers."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        lens = [int(x) for x in rng.integers(0, 5000, size=int(rng.integers(1, 7)))]
        W = int(rng.integers(1, 40))
        mp = parse_map(ref_plan(lens, W, 512))
        got = []
        for w in range(W):
            got.append(sum(-(-(int(e) - int(a)) // 512) for _, _, a, e in mp.worker_segments(w)))
        T = sum(-(-L // 512) for L in lens)
        base, rem = T // W, T % W
        assert got == [base + 1] * rem + [base] * (W - rem), (lens, W, got)


# ------------------------------------------------------------------------------------------------
# 8-bit (E4M3) KV cache.

def _torch_e4m3_values():
    """Every E4M3 code through torch's own float8_e4m3fn conversion (a library routine)."""
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_e4m3_library(e4m3_table):
    """All 256 codes agree with torch's float8_e4m3fn decoding, NaN codes included."""
    got = np.asarray(e4m3_table(), dtype=np.float64)
    exp = _torch_e4m3_values()
    assert got.shape == (256,)
    assert np.array_equal(np.isnan(got), np.isnan(exp))
    fin = ~np.isnan(exp)
    assert np.array_equal(got[fin], exp[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(exp[fin]))


def pin_e4m3_closed_forms(e4m3_value):
    """Values the OCP E4M3 definition fixes: one, the largest finite value, the smallest
    subnormal and normal, signed zero, and the two NaN codes."""
    fixed = {0x00: 0.0, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x08: 2.0 ** -6, 0x30: 0.5, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for code, val in fixed.items():
        assert e4m3_value(code) == val, (hex(code), e4m3_value(code), val)
    assert math.copysign(1.0, e4m3_value(0x80)) == -1.0 and e4m3_value(0x80) == 0.0
    assert math.isnan(e4m3_value(0x7F)) and math.isnan(e4m3_value(0xFF))
    vals = [e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:])), "positive codes must increase"
    for c in range(0x7F):
        assert e4m3_value(c | 0x80) == -vals[c]


def pin_fp8_decode_library(ref_decode_fp8):
    """Decode over an FP8 cache equals torch's SDPA (float64) over torch-dequantised K and V."""
    g = torch.Generator().manual_seed(11)
    for (L, Hq, Hkv, D) in [(9, 8, 2, 16), (1, 4, 4, 8), (17, 8, 1, 32)]:
        q = torch.randn(2, Hq, D, generator=g).to(torch.bfloat16).to(torch.float64)
        kc = [torch.randint(0, 256, (L, Hkv, D), generator=g, dtype=torch.int32).to(torch.uint8) for _ in range(2)]
        vc = [torch.randint(0, 256, (L, Hkv, D), generator=g, dtype=torch.int32).to(torch.uint8) for _ in range(2)]
        for c in kc + vc:   # no NaN codes in a stored cache
            c[(c & 0x7F) == 0x7F] = 0x3A
        ks = (0.01 + torch.rand(Hkv, generator=g, dtype=torch.float64)).to(torch.float32).to(torch.float64)
        vs = (0.01 + torch.rand(Hkv, generator=g, dtype=torch.float64)).to(torch.float32).to(torch.float64)
        got = ref_decode_fp8(q.numpy(), [c.numpy() for c in kc], [c.numpy() for c in vc], ks.numpy(), vs.numpy(), 0.3)
        per = Hq // Hkv
        for b in range(2):
            k = kc[b].view(torch.float8_e4m3fn).to(torch.float64) * ks[None, :, None]
            v = vc[b].view(torch.float8_e4m3fn).to(torch.float64) * vs[None, :, None]
            kk = k.repeat_interleave(per, dim=1).permute(1, 0, 2)
            vv = v.repeat_interleave(per, dim=1).permute(1, 0, 2)
            exp = torch.nn.functional.scaled_dot_product_attention(
                q[b:b + 1].permute(1, 0, 2), kk, vv, scale=0.3).permute(1, 0, 2).numpy()[0]
            assert np.allclose(got[b], exp, rtol=1e-12, atol=1e-12)


def pin_fp8_scale_laws(ref_decode_fp8):
    """Scaling every K scale by c equals scaling the softmax scale by c; scaling every V scale by c
    scales the output by c; a single key returns its dequantised value row."""
    rng = np.random.default_rng(12)
    Hq, Hkv, D, L = 8, 2, 16, 11
    q = rng.standard_normal((1, Hq, D))
    kc = [rng.integers(0, 0x7F, (L, Hkv, D), dtype=np.uint8)]
    vc = [rng.integers(0, 0x7F, (L, Hkv, D), dtype=np.uint8) | (rng.integers(0, 2, (L, Hkv, D), dtype=np.uint8) << 7)]
    ks, vs = np.array([0.011, 0.023]), np.array([0.5, 0.125])
    base = ref_decode_fp8(q, kc, vc, ks, vs, 0.2)
    assert np.allclose(ref_decode_fp8(q, kc, vc, 3 * ks, vs, 0.2), ref_decode_fp8(q, kc, vc, ks, vs, 0.6),
                       rtol=1e-12, atol=1e-14)
    assert not np.allclose(ref_decode_fp8(q, kc, vc, 3 * ks, vs, 0.2), base, rtol=1e-6, atol=1e-9)
    assert np.allclose(ref_decode_fp8(q, kc, vc, ks, 4 * vs, 0.2), 4 * base, rtol=1e-12, atol=1e-14)
    one = ref_decode_fp8(q, [kc[0][:1]], [vc[0][:1]], ks, vs, 0.2)[0]
    exp = _torch_e4m3_values()[vc[0][0]] * vs[:, None]            # [Hkv, D]
    assert np.array_equal(one, np.repeat(exp, Hq // Hkv, axis=0))


# ------------------------------------------------------------------------------------------------
# LPT comparison planner.

def _lpt_worker_tiles(ref_plan_lpt, parse_map, lens, W, tile):
    mp = parse_map(ref_plan_lpt(lens, W, tile))
    assert mp.version == 2 and sorted(mp.order.tolist()) == list(range(mp.S))
    per = []
    for w in range(W):
        tiles = []
        for b, qt, a, e in mp.worker_segments(w).tolist():
            assert qt == 0 and 0 <= a < e <= lens[b] and a % tile == 0
            tiles += [(b, t) for t in range(a // tile, -(-e // tile))]
        per.append(tiles)
    # slots are unit-major and each unit's slots are contiguous
    for u in range(mp.U):
        assert all(s[0] == u for s in mp.unit_segments(u).tolist())
    return mp, per


def pin_lpt_coverage_and_balance(ref_plan_lpt, parse_map, trials=120, seed=9):
    """Every tile on exactly one worker; max load - min load <= the largest tile (the greedy
    least-loaded rule guarantees it); loads counted in tokens."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        B = int(rng.integers(0, 9))
        W = int(rng.integers(1, 9))
        tile = int(rng.choice([16, 64, 512]))
        lens = [int(x) for x in rng.integers(0, 3000, size=B)]
        mp, per = _lpt_worker_tiles(ref_plan_lpt, parse_map, lens, W, tile)
        seen = sorted(t for tiles in per for t in tiles)
        expect = sorted((b, t) for b, L in enumerate(lens) for t in range(-(-L // tile) if L > 0 else 0))
        assert seen == expect
        size = lambda bt: min(tile, lens[bt[0]] - bt[1] * tile)
        loads = [sum(size(bt) for bt in tiles) for tiles in per]
        if expect:
            assert max(loads) - min(loads) <= max(size(bt) for bt in expect)


def pin_lpt_equal_sizes_round_robin(ref_plan_lpt, parse_map):
    """With every tile full-size, decreasing size keeps stream order and each tile goes to the least
    loaded (lowest-index) worker: stream tile j lands on worker j mod W."""
    for lens, W in (([1024, 5120, 2048], 4), ([512 * 7, 512 * 3], 3), ([2048] * 5, 7)):
        _, per = _lpt_worker_tiles(ref_plan_lpt, parse_map, lens, W, 512)
        stream = [(b, t) for b, L in enumerate(lens) for t in range(L // 512)]
        for j, bt in enumerate(stream):
            assert bt in per[j % W], (lens, W, j)
    # one worker: every request's tiles are consecutive there and merge into one segment
    mp, _ = _lpt_worker_tiles(ref_plan_lpt, parse_map, [1024, 5120, 0, 2048], 1, 512)
    assert mp.S == 3 and mp.segs.tolist() == [[0, 0, 0, 1024], [1, 0, 0, 5120], [3, 0, 0, 2048]]


def pin_lpt_hand_example(ref_plan_lpt, parse_map):
    """Lengths 700, 1500, 0, 300 with 512-token tiles on 3 workers, worked by hand: tile sizes
    512 (0:0), 188 (0:1), 512 (1:0), 512 (1:1), 476 (1:2), 300 (3:0); in decreasing size
    0:0 -> w0, 1:0 -> w1, 1:1 -> w2, 1:2 -> w0 (988), 3:0 -> w1 (812), 0:1 -> w2 (700)."""
    _, per = _lpt_worker_tiles(ref_plan_lpt, parse_map, [700, 1500, 0, 300], 3, 512)
    assert [sorted(p) for p in per] == [[(0, 0), (1, 2)], [(1, 0), (3, 0)], [(0, 1), (1, 1)]]
    # loads are tokens, not tiles: lengths 512, 100, 100, 100 on 2 workers put the 512-token tile
    # alone on w0 (512) and the three 100-token tiles on w1 (100, 200, 300 < 512)
    _, per = _lpt_worker_tiles(ref_plan_lpt, parse_map, [512, 100, 100, 100], 2, 512)
    assert [sorted(p) for p in per] == [[(0, 0)], [(1, 0), (2, 0), (3, 0)]]


# ------------------------------------------------------------------------------------------------
# Cost-weighted comparison planner.

def _weighted_worker_tiles(ref_plan_weighted, parse_map, lens, W, tile, split_cost):
    mp = parse_map(ref_plan_weighted(lens, W, tile, split_cost))
    assert mp.version == 1
    per = []
    for w in range(W):
        tiles = []
        for b, qt, a, e in mp.worker_segments(w).tolist():
            assert qt == 0 and 0 <= a < e <= lens[b] and a % tile == 0 and (e % tile == 0 or e == lens[b])
            tiles += [(b, t) for t in range(a // tile, -(-e // tile))]
        per.append(tiles)
    return mp, per


def pin_weighted_contiguous_and_balanced(ref_plan_weighted, parse_map, trials=150, seed=11):
    """The workers' tiles read in worker order are the task stream itself (a contiguous fill: no tile
    lost, repeated or reordered); each worker holds one segment per request it touches; and every
    worker's cost is within the largest tile cost of C / W.  The bound follows from the midpoint
    rule: worker w's share [wC/W, (w+1)C/W) of the cost line is covered by its own tiles plus at most
    half a tile at each end, and its own tiles reach at most half a tile beyond it on each side."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        B = int(rng.integers(0, 10))
        W = int(rng.integers(1, 10))
        tile = int(rng.choice([64, 128, 512]))
        sc = int(rng.choice([0, 1, 64, 300, 2000]))
        lens = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 4000, size=B)]
        mp, per = _weighted_worker_tiles(ref_plan_weighted, parse_map, lens, W, tile, sc)
        stream = [(b, t) for b, L in enumerate(lens) for t in range(-(-L // tile))]
        assert [x for tiles in per for x in tiles] == stream
        assert mp.T == len(stream)
        assert mp.S == sum(len({b for b, _ in tiles}) for tiles in per)
        if not stream:
            continue
        cost = lambda bt: min(tile, lens[bt[0]] - bt[1] * tile) + (sc if bt[1] == 0 else 0)
        C = sum(cost(x) for x in stream)
        cmax = max(cost(x) for x in stream)
        for tiles in per:
            cw = sum(cost(x) for x in tiles)
            assert C - W * cmax <= W * cw <= C + W * cmax, (lens, W, tile, sc)


def pin_weighted_worked_example(ref_plan_weighted, parse_map):
    """With no split cost and whole tiles every tile costs the same, and the pages' worked example
    (lengths 1024, 5120, 2048; 512-token tiles; 4 workers) again gives 4 tiles per worker with the
    long request spread over workers — the same map as the pages' fill."""
    ex = load_worked_example()
    _, per = _weighted_worker_tiles(ref_plan_weighted, parse_map, ex["seq_lens"], ex["num_workers"], ex["tile"], 0)
    assert [len(t) for t in per] == ex["tiles_per_worker"]
    assert len({w for w, tiles in enumerate(per) for b, _ in tiles if b == 1}) > 1


def pin_weighted_hand_examples(ref_plan_weighted, parse_map):
    """Worked by hand (c = tile cost, mid = cost before the tile + c / 2, worker = floor(W mid / C)):
    (a) 512, 100, 100, 100 on 2 workers: c = 512, 100, 100, 100, C = 812, mids 256, 562, 662, 762
        -> workers 0, 1, 1, 1 (a tile count would pair the 512-token tile with a 100-token one);
    (b) 512, 512, 10, 10 on 2 workers: split cost 0 -> C = 1044, mids 256, 768, 1029, 1039 -> 0, 1, 1, 1;
        split cost 500 -> c = 1012, 1012, 510, 510, C = 3044, mids 506, 1518, 2279, 2789 -> 0, 0, 1, 1;
    (c) 700, 1500, 0, 300 on 3 workers, 512-token tiles: c = 512, 188 | 512, 512, 476 | 300, C = 2500,
        mids 256, 606, 956, 1468, 1962, 2350 -> 0, 0, 1, 1, 2, 2: worker loads 700, 1024, 776;
    (d) 4096 then eight 64-token requests on 2 workers, split cost 512: the long request costs
        4096 + 512 = 4608 and the eight short ones 8 x 576 = 4608, C = 9216; its last tile's mid is
        4352 < 4608 and the first short one's 4896 -> the long request alone on worker 0."""
    f = lambda lens, W, sc: [sorted(t) for t in _weighted_worker_tiles(ref_plan_weighted, parse_map, lens, W, 512, sc)[1]]
    assert f([512, 100, 100, 100], 2, 0) == [[(0, 0)], [(1, 0), (2, 0), (3, 0)]]
    assert f([512, 512, 10, 10], 2, 0) == [[(0, 0)], [(1, 0), (2, 0), (3, 0)]]
    assert f([512, 512, 10, 10], 2, 500) == [[(0, 0), (1, 0)], [(2, 0), (3, 0)]]
    assert f([700, 1500, 0, 300], 3, 0) == [[(0, 0), (0, 1)], [(1, 0), (1, 1)], [(1, 2), (3, 0)]]
    mp, _ = _weighted_worker_tiles(ref_plan_weighted, parse_map, [700, 1500, 0, 300], 3, 512, 0)
    assert mp.segs.tolist() == [[0, 0, 0, 700], [1, 0, 0, 1024], [1, 0, 1024, 1500], [3, 0, 0, 300]]
    assert f([4096] + [64] * 8, 2, 512) == [[(0, t) for t in range(8)], [(b, 0) for b in range(1, 9)]]


# ------------------------------------------------------------------------------------------------
# Rate-proportional planner.

def _rated_worker_tiles(ref_plan_rated, parse_map, lens, W, tile, split_cost, rates):
    mp = parse_map(ref_plan_rated(lens, W, tile, split_cost, rates))
    assert mp.version == 3
    per = []
    for w in range(W):
        tiles = []
        for b, qt, a, e in mp.worker_segments(w).tolist():
            assert qt == 0 and 0 <= a < e <= lens[b] and a % tile == 0 and (e % tile == 0 or e == lens[b])
            tiles += [(b, t) for t in range(a // tile, -(-e // tile))]
        per.append(tiles)
    return mp, per


def pin_rated_equal_rates_are_weighted(ref_plan_rated, ref_plan_weighted, trials=120, seed=13):
    """Equal rates, whatever their common value, give the cost-weighted map word for word apart from
    the version word: the share boundaries C w r / (W r) are the equal shares."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        B = int(rng.integers(0, 10))
        W = int(rng.integers(1, 12))
        tile = int(rng.choice([64, 128, 512]))
        sc = int(rng.choice([0, 1, 64, 300, 2000]))
        r = int(rng.choice([1, 7, 1000, 1 << 20]))
        lens = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 4000, size=B)]
        got = ref_plan_rated(lens, W, tile, sc, [r] * W)
        want = ref_plan_weighted(lens, W, tile, sc)
        assert got[0] == 3 and want[0] == 1
        assert np.array_equal(got[1:], want[1:]), (lens, W, tile, sc, r)


def pin_rated_contiguous_and_proportional(ref_plan_rated, parse_map, trials=150, seed=17):
    """The workers' tiles read in worker order are the task stream itself (no tile lost, repeated or
    reordered); each worker holds one segment per request it touches; a worker of rate 0 gets no
    tile; and every worker's cost is within the largest tile cost of C r_w / R — its share of the
    cost line is covered by its own tiles up to half a tile at each end, and its tiles reach at most
    half a tile beyond it on each side."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        B = int(rng.integers(0, 10))
        W = int(rng.integers(1, 10))
        tile = int(rng.choice([64, 128, 512]))
        sc = int(rng.choice([0, 1, 64, 300, 2000]))
        rates = [int(x) if rng.random() > 0.2 else 0 for x in rng.integers(1, 100, size=W)]
        if sum(rates) == 0:
            rates[int(rng.integers(0, W))] = 1
        lens = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 4000, size=B)]
        mp, per = _rated_worker_tiles(ref_plan_rated, parse_map, lens, W, tile, sc, rates)
        stream = [(b, t) for b, L in enumerate(lens) for t in range(-(-L // tile))]
        assert [x for tiles in per for x in tiles] == stream
        assert mp.T == len(stream)
        assert mp.S == sum(len({b for b, _ in tiles}) for tiles in per)
        assert all(not tiles for tiles, r in zip(per, rates) if r == 0)
        if not stream:
            continue
        cost = lambda bt: min(tile, lens[bt[0]] - bt[1] * tile) + (sc if bt[1] == 0 else 0)
        C = sum(cost(x) for x in stream)
        cmax = max(cost(x) for x in stream)
        R = sum(rates)
        for tiles, r in zip(per, rates):
            cw = sum(cost(x) for x in tiles)
            assert abs(R * cw - C * r) <= R * cmax, (lens, W, tile, sc, rates)


def pin_rated_hand_examples(ref_plan_rated, parse_map):
    """Worked by hand (c = tile cost, mid = cost before the tile + c / 2, worker w's share
    [C R_w / R, C R_(w+1) / R)):
    (a) the worked example's lengths 1024, 5120, 2048 (512-token tiles) on rates 1 and 3: C = 8192,
        worker 1's share starts at 2048, mids 256 + 512 i -> tiles 0-3 of the stream on worker 0,
        the other 12 on worker 1;
    (b) six 512-token requests on rates 1, 0, 2: C = 3072, shares [0, 1024), empty, [1024, 3072)
        -> requests 0-1 on worker 0, none on worker 1, 2-5 on worker 2;
    (c) two 4096-token requests, 64-token tiles, rates 20, 19, 20, 19: C = 8192, R = 78, shares
        start at 0, 2100.5, 4096, 6196.5; mids 32 + 64 i -> 33, 31, 33, 31 tiles;
    (d) 512, 512, 10, 10 with split cost 500 on rates 1 and 2: c = 1012, 1012, 510, 510, C = 3044,
        worker 1 from 1014.7, mids 506, 1518, 2279, 2789 -> 0, 1, 1, 1 (equal rates: 0, 0, 1, 1);
    (e) a midpoint exactly on a share boundary goes to the later worker: one 1536-token request on
        two workers of rate 5, C = 1536, boundary 768, mids 256, 768, 1280 -> 0, 1, 1."""
    f = lambda lens, W, tile, sc, rates: _rated_worker_tiles(ref_plan_rated, parse_map, lens, W, tile, sc, rates)[1]
    stream = [(0, 0), (0, 1)] + [(1, t) for t in range(10)] + [(2, t) for t in range(4)]
    assert f([1024, 5120, 2048], 2, 512, 0, [1, 3]) == [stream[:4], stream[4:]]
    assert f([512] * 6, 3, 512, 0, [1, 0, 2]) == [[(0, 0), (1, 0)], [], [(b, 0) for b in range(2, 6)]]
    assert [len(t) for t in f([4096, 4096], 4, 64, 0, [20, 19, 20, 19])] == [33, 31, 33, 31]
    assert f([512, 512, 10, 10], 2, 512, 500, [1, 2]) == [[(0, 0)], [(1, 0), (2, 0), (3, 0)]]
    assert f([512, 512, 10, 10], 2, 512, 500, [1, 1]) == [[(0, 0), (1, 0)], [(2, 0), (3, 0)]]
    assert f([1536], 2, 512, 0, [5, 5]) == [[(0, 0)], [(0, 1), (0, 2)]]
    mp, _ = _rated_worker_tiles(ref_plan_rated, parse_map, [1024, 5120, 2048], 2, 512, 0, [1, 3])
    assert mp.segs.tolist() == [[0, 0, 0, 1024], [1, 0, 0, 1024], [1, 0, 1024, 5120], [2, 0, 0, 2048]]
    assert mp.worker_ptr.tolist() == [0, 2, 4]


# ------------------------------------------------------------------------------------------------
# Producer step (normalise, rotate, quantise, store).

def pin_round_bf16_library(round_bf16):
    """bf16 rounding of float32 inputs equals torch's float32 -> bfloat16 conversion (RNE)."""
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.standard_normal(50000) * 3, rng.standard_normal(2000) * 1e-30,
                        [0.0, -0.0, 1.0, -1.5, 1.00390625, 1.005859375]]).astype(np.float32)
    # exact ties: a bf16 value plus half of its step (8 significant bits)
    t = torch.randn(3000, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).to(torch.float32).numpy()
    m, e = np.frexp(t.astype(np.float64))
    x = np.concatenate([x, (t + np.ldexp(1.0, e - 9)).astype(np.float32)])
    got = round_bf16(x.astype(np.float64))
    exp = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, exp)


def pin_e4m3_round_library(e4m3_round, e4m3_table):
    """E4M3 rounding of float32 inputs in [-448, 448] equals torch's float8_e4m3fn conversion, exact
    ties (midpoints of neighbouring codes) included."""
    rng = np.random.default_rng(32)
    x = np.concatenate([rng.standard_normal(40000) * 60, rng.uniform(-448, 448, 20000),
                        rng.standard_normal(5000) * 1e-3, [0.0, 448.0, -448.0, 1e-9, -1e-9]])
    vals = e4m3_table()[np.arange(0x00, 0x7F)]
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    x = np.clip(x, -448, 448)
    got = e4m3_round(x.astype(np.float64))
    exp = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, exp), int((got != exp).sum())


def pin_hadamard(hadamard):
    """Against scipy's Hadamard matrix; an involution (H / sqrt(n) is symmetric and orthogonal)."""
    import scipy.linalg
    for n in (1, 2, 8, 128):
        assert np.allclose(hadamard(np.eye(n)), scipy.linalg.hadamard(n) / math.sqrt(n), atol=1e-15)
    x = np.random.default_rng(33).standard_normal((5, 128))
    assert np.allclose(hadamard(hadamard(x)), x, atol=1e-12)


def pin_rope(rope):
    """Closed forms: position 0 is the identity; (1, 0, 0, 0) at position 1 with theta 10000 and D 4
    turns into (cos 1, 0, sin 1, 0) (pair (0, 2) at frequency 1) and (0, 1, 0, 0) at position 100
    into (0, cos 1, 0, sin 1) (pair (1, 3) at frequency 0.01); each pair keeps its length; and
    <rope(q, p), rope(k, r)> depends on p - r only (the relative-position property)."""
    rng = np.random.default_rng(34)
    x = rng.standard_normal((3, 2, 16))
    assert np.allclose(rope(x, np.zeros(3), 10000.0), x, atol=1e-15)
    one = rope(np.array([[[1.0, 0.0, 0.0, 0.0]]]), np.array([1.0]), 10000.0)[0, 0]
    assert np.allclose(one, [math.cos(1.0), 0.0, math.sin(1.0), 0.0], atol=1e-15)
    # pair (1, 3) turns at 10000^(-2/4) = 0.01 per position: position 100 -> angle 1
    two = rope(np.array([[[0.0, 1.0, 0.0, 0.0]]]), np.array([100.0]), 10000.0)[0, 0]
    assert np.allclose(two, [0.0, math.cos(1.0), 0.0, math.sin(1.0)], atol=1e-12)
    y = rope(x, np.array([5.0, 77.0, 123456.0]), 10000.0)
    assert np.allclose(x[..., :8] ** 2 + x[..., 8:] ** 2, y[..., :8] ** 2 + y[..., 8:] ** 2, atol=1e-12)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    d1 = np.sum(rope(q, np.array([10.0]), 500.0) * rope(k, np.array([3.0]), 500.0))
    d2 = np.sum(rope(q, np.array([1010.0]), 500.0) * rope(k, np.array([1003.0]), 500.0))
    assert abs(d1 - d2) < 1e-9


def pin_rms_norm_library(rms_norm):
    """Against torch.nn.functional.rms_norm in float64."""
    rng = np.random.default_rng(35)
    x = rng.standard_normal((4, 3, 128)) * 5
    w = rng.standard_normal(128)
    exp = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps=1e-6).numpy()
    assert np.allclose(rms_norm(x, w, 1e-6), exp, rtol=1e-12, atol=1e-12)


def pin_store_kv_scores_invariant(ref_store_kv):
    """The Hadamard step rotates q and k alike, so every q.k is unchanged (before rounding)."""
    from oracle import store_kv as SK
    rng = np.random.default_rng(36)
    q = rng.standard_normal((2, 16, 128))
    k = rng.standard_normal((2, 2, 128))
    pos = np.array([7.0, 300.0])
    a = SK.rope(q, pos, 10000.0), SK.rope(k, pos, 10000.0)
    s1 = np.einsum("nhd,ngd->nhg", a[0], a[1])
    s2 = np.einsum("nhd,ngd->nhg", SK.hadamard(a[0]), SK.hadamard(a[1]))
    assert np.allclose(s1, s2, atol=1e-10)
    # and the full step with Hadamard on matches the library pieces composed by hand
    qo, ko, vo = ref_store_kv(q, k, k, pos, None, None, 1e-6, 10000.0, True)
    assert np.array_equal(qo, SK.round_bf16(SK.hadamard(a[0])))
    assert np.array_equal(ko, SK.round_bf16(SK.hadamard(a[1])))


def _assert_bf16_nearest(got, exact, what):
    """got holds bf16 values (torch's float32 -> bfloat16 round trip leaves them unchanged) within
    half a bf16 step (8 significant bits) of the exact value: what round-to-nearest must give."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    rt = torch.from_numpy(got.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rt, got), f"{what}: not bf16 values"
    _, e = np.frexp(exact)
    half_step = np.ldexp(1.0, e - 9)
    bad = np.abs(got - exact) > half_step * (1 + 1e-9) + 1e-300
    assert not bad.any(), f"{what}: {int(bad.sum())} values off by more than half a bf16 step"


def _sylvester_sign(i, j):
    """Entry (i, j) of the Sylvester-ordered Hadamard matrix: (-1)^popcount(i & j)."""
    return -1.0 if bin(i & j).count("1") % 2 else 1.0


def pin_store_kv_composition(ref_store_kv):
    """Which vector takes which step, with which gain and scale, in which order — closed forms worked
    out by hand and run through the whole producer step ([P3] §4.1: RoPE, RMSNorm, Hadamard,
    quantisation and store fused; §8: q and k rotated before the 8-bit code).

    (a) v is stored as given (rounded to bf16, or e4m3(v / v_scale[head])) whatever theta, gains
        and Hadamard are: bf16 v comes back bit for bit; v = s 2^j v_scale[g] stores the code of
        s 2^j (exponent field j + 7, mantissa 0, sign bit for s < 0).
    (b) Gains reach their own kind only: x = c 1 with c = +-2^j and eps = 0 normalises to
        sign(c) 1 exactly, so q comes out as sign(c) q_norm_w and k as sign(c) k_norm_w.
    (c) eps sits under the root, added to the mean square: x = 1, eps = 3 gives w / 2.
    (d) Position 0 is the identity of RoPE at any theta.
    (e) A one-hot e_j through the Hadamard gives (-1)^popcount(i & j) / sqrt(128) at dim i.
    (f) Order RMSNorm -> RoPE -> Hadamard: x = c 1 with gain e_0 normalises to sign(c) e_0; RoPE at
        position p turns the pair (0, 64) at frequency 1, giving sign(c) (cos p e_0 + sin p e_64);
        the Hadamard then gives sign(c) (cos p + sin p s_i) / sqrt(128), s_i = +1 below dim 64 and
        -1 from it (column 64 of the Sylvester matrix).
    (g) k takes k_scale: k = c 1 (c = +-2^j) with gain 2^-m 1, eps = 0, position 0 and the Hadamard
        on becomes sign(c) 2^-m sqrt(128) e_0 (H 1 / sqrt(128) = sqrt(128) e_0); with k_scale[g] =
        2^-m sqrt(128) / 2^(g+1) its code at dim 0 is that of sign(c) 2^(g+1), zero elsewhere."""
    rng = np.random.default_rng(37)
    D, N, Hq, Hkv = 128, 3, 16, 2
    bf = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    pos_big = np.array([5.0, 4097.0, 123457.0])
    zero_pos = np.zeros(N)
    qw = bf(1 + 0.3 * rng.standard_normal(D))
    kw = bf(-1 + 0.3 * rng.standard_normal(D))

    def e4m3_pow2(s, j):
        return np.where(s < 0, 0x80, 0x00) | ((j + 7) << 3)

    # (a) v untouched by norm, RoPE and Hadamard; v_scale (not k_scale) sets its code
    q = bf(rng.standard_normal((N, Hq, D)))
    k = bf(rng.standard_normal((N, Hkv, D)))
    v = bf(rng.standard_normal((N, Hkv, D)) * 3)
    for theta, had in ((10000.0, True), (1e6, False), (0.0, True)):
        _, _, vo = ref_store_kv(q, k, v, pos_big, qw, kw, 1e-6, theta, had)
        assert np.array_equal(vo, v), "(a) v changed by the q/k steps"
    k_scale = np.array([2.0 ** -3, 2.0 ** -1])
    v_scale = np.array([2.0 ** -6, 2.0 ** 2])
    jv = rng.integers(-3, 8, size=(N, Hkv, D))
    sv = np.where(rng.random((N, Hkv, D)) < 0.5, -1.0, 1.0)
    v8 = sv * np.ldexp(1.0, jv) * v_scale[None, :, None]
    _, _, vc = ref_store_kv(q, k, v8, pos_big, qw, kw, 1e-6, 10000.0, True, k_scale, v_scale)
    assert np.array_equal(vc.astype(np.int64), e4m3_pow2(sv, jv)), "(a) v code not e4m3(v / v_scale)"

    # (b) gains reach their own kind only
    cq = np.where(rng.random((N, Hq, 1)) < 0.5, -1.0, 1.0) * np.ldexp(1.0, rng.integers(-4, 5, (N, Hq, 1)))
    ck = np.where(rng.random((N, Hkv, 1)) < 0.5, -1.0, 1.0) * np.ldexp(1.0, rng.integers(-4, 5, (N, Hkv, 1)))
    qo, ko, _ = ref_store_kv(cq * np.ones(D), ck * np.ones(D), v, pos_big, qw, kw, 0.0, 0.0, False)
    assert np.array_equal(qo, np.sign(cq) * qw), "(b) q does not carry sign(c) q_norm_w"
    assert np.array_equal(ko, np.sign(ck) * kw), "(b) k does not carry sign(c) k_norm_w"
    qo, ko, _ = ref_store_kv(cq * np.ones(D), ck * np.ones(D), v, pos_big, None, kw, 0.0, 0.0, False)
    assert np.array_equal(qo, cq * np.ones(D)) and np.array_equal(ko, np.sign(ck) * kw), "(b) q normalised without a gain"

    # (c) eps under the root
    qo, ko, _ = ref_store_kv(np.ones((N, Hq, D)), np.ones((N, Hkv, D)), v, pos_big, qw, kw, 3.0, 0.0, False)
    assert np.array_equal(qo, np.broadcast_to(qw / 2, qo.shape)) and np.array_equal(ko, np.broadcast_to(kw / 2, ko.shape)), "(c) eps"

    # (d) position 0: RoPE is the identity for q and k
    qo, ko, vo = ref_store_kv(q, k, v, zero_pos, None, None, 1e-6, 10000.0, False)
    assert np.array_equal(qo, q) and np.array_equal(ko, k) and np.array_equal(vo, v), "(d) position 0"

    # (e) one-hot vectors through the Hadamard, q and k alike
    js = [0, 1, 5, 64, 127, 85]
    for j in js:
        e = np.zeros(D)
        e[j] = 1.0
        col = np.array([_sylvester_sign(i, j) for i in range(D)]) / math.sqrt(D)
        qo, ko, _ = ref_store_kv(np.broadcast_to(e, (N, Hq, D)), np.broadcast_to(-e, (N, Hkv, D)), v, zero_pos,
                                 None, None, 1e-6, 0.0, True)
        _assert_bf16_nearest(qo, np.broadcast_to(col, qo.shape), f"(e) q one-hot {j}")
        _assert_bf16_nearest(ko, np.broadcast_to(-col, ko.shape), f"(e) k one-hot {j}")

    # (f) order: RMSNorm, then RoPE, then Hadamard
    e0 = np.zeros(D)
    e0[0] = 1.0
    s = np.where(np.arange(D) < 64, 1.0, -1.0)
    p = np.array([3.0, 1.0, 2.0])
    for had in (False, True):
        qo, ko, _ = ref_store_kv(cq * np.ones(D), ck * np.ones(D), v, p, e0, e0, 0.0, 10000.0, had)
        for got, c, what in ((qo, cq, "q"), (ko, ck, "k")):
            cos, sin = np.cos(p)[:, None, None], np.sin(p)[:, None, None]
            if had:
                exact = np.sign(c) * (cos + sin * s) / math.sqrt(D)
            else:
                exact = np.zeros(got.shape)
                exact[..., 0:1] = np.sign(c) * cos
                exact[..., 64:65] = np.sign(c) * sin
            _assert_bf16_nearest(got, np.broadcast_to(exact, got.shape), f"(f) {what} order, hadamard={had}")

    # (g) k takes k_scale (per head) after its own steps
    m = 3
    kg = np.full(D, 2.0 ** -m)
    k_scale_g = np.array([2.0 ** -m * math.sqrt(D) / 2.0 ** (g + 1) for g in range(Hkv)])
    _, kc, _ = ref_store_kv(q, ck * np.ones(D), v8, zero_pos, None, kg, 0.0, 10000.0, True, k_scale_g, v_scale)
    want = np.zeros((N, Hkv, D), dtype=np.int64)
    want[..., 0] = e4m3_pow2(np.sign(ck[..., 0]), np.arange(Hkv)[None, :] + 1)
    assert np.array_equal(kc.astype(np.int64), want), "(g) k code not e4m3(k / k_scale) of the processed k"
