"""Seeded random sweep of the GPU paths against the fp64 oracle.  Each case draws its own
configuration from its seed, so the sweep crosses options the hand-picked cases take one at a time:
decode (planner greedy / LPT / cost-weighted, and rate-proportional with random rates, workers, head
groups, tile 64-1024, page 64-256, bf16 or E4M3 cache, empty requests), chunked prefill (unit height, P.V mode, causal or not, KV tile,
page) and multi-token decode (0-4 rows, bf16 or E4M3, page).  Pads and partial buffers hold NaN, so a
read outside a request's keys or a slot the combine should not touch shows up in the output."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import (SCALE, assert_close, decode_inputs, decode_inputs_fp8, mtp_inputs, note, oracle_decode,
                         oracle_decode_fp8, oracle_mtp, prefill_inputs, q_starts)
from oracle.attention import ref_attention
from oracle.plan import ref_plan, ref_plan_lpt, ref_plan_prefill, ref_plan_rated, ref_plan_weighted

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _rng(kind: int, seed: int) -> np.random.Generator:
    return np.random.default_rng([kind, seed])


@pytest.mark.parametrize("seed", range(64))
def test_decode_sweep(lb, seed):
    g = _rng(1, seed)
    batch = int(g.integers(1, 10))
    max_len = int(g.choice([200, 1000, 3000, 6000]))
    wl = WL.random_decode(600 + seed, batch, max_len)
    if g.random() < 0.3:
        wl.kv_lens[int(g.integers(0, batch))] = 0
    W = int(g.integers(1, 41))
    G = int(g.choice([1, 2, 4, 8]))
    tile = int(g.choice([64, 128, 256, 512, 1024]))
    page = int(g.choice([64, 128, 256]))
    fp8 = bool(g.random() < 0.5)
    planner = str(g.choice(["greedy", "lpt", "weighted"]))
    note(f"decode sweep {seed}: lens={wl.kv_lens} W={W} G={G} tile={tile} page={page} fp8={fp8} planner={planner}")
    if planner == "greedy":
        words, ref_words = lb.attn_plan(wl.kv_lens, W, tile), ref_plan(wl.kv_lens, W, tile)
    elif planner == "lpt":
        words, ref_words = lb.attn_plan_lpt(wl.kv_lens, W, tile), ref_plan_lpt(wl.kv_lens, W, tile)
    else:
        cost = int(g.choice([0, 64, 512]))
        words = lb.attn_plan_weighted(wl.kv_lens, W, tile, cost)
        ref_words = ref_plan_weighted(wl.kv_lens, W, tile, cost)
    assert np.array_equal(words, ref_words)
    _run_decode_case(lb, wl, words, G, page, fp8, f"decode sweep {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_decode_sweep_rated(lb, seed):
    """Rate-proportional (version-3, list-major) maps with random rates, zeros included."""
    g = _rng(4, seed)
    batch = int(g.integers(1, 10))
    max_len = int(g.choice([200, 1000, 3000, 6000]))
    wl = WL.random_decode(900 + seed, batch, max_len)
    if g.random() < 0.3:
        wl.kv_lens[int(g.integers(0, batch))] = 0
    W = int(g.choice([8, 16, 24, int(g.integers(1, 41))]))
    G = int(g.choice([1, 2, 4, 8]))
    tile = int(g.choice([64, 128, 256, 512, 1024]))
    page = int(g.choice([64, 128, 256]))
    fp8 = bool(g.random() < 0.5)
    cost = int(g.choice([0, 64, 512]))
    rates = [int(r) if g.random() > 0.2 else 0 for r in g.integers(1, 1 << 16, size=W)]
    if sum(rates) == 0:
        rates[0] = 1
    note(f"rated sweep {seed}: lens={wl.kv_lens} W={W} G={G} tile={tile} page={page} fp8={fp8} cost={cost} "
         f"rates={rates}")
    words = lb.attn_plan_rated(wl.kv_lens, W, rates, tile, cost)
    assert np.array_equal(words, ref_plan_rated(wl.kv_lens, W, tile, cost, rates))
    _run_decode_case(lb, wl, words, G, page, fp8, f"rated sweep {seed}")


def _run_decode_case(lb, wl, words, G, page, fp8, what):
    """One decode step over `words` with NaN in the pads and partial buffers, against the oracle."""
    from load_balanced_split_attn_amd import map_header
    if fp8:
        inputs = decode_inputs_fp8(wl, page=page, pad_code=NAN_CODE)
        ref = oracle_decode_fp8(wl)
    else:
        inputs = decode_inputs(wl, page=page, pad_value=float("nan"))
        ref = oracle_decode(wl)
    q, kc, vc, bt = inputs[:4]
    dev = q.device
    hdr = map_header(words)
    mp = torch.from_numpy(np.asarray(words, dtype=np.int32)).to(dev)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    S = max(hdr["S"], 1)
    pm = torch.full((S, wl.hq), float("nan"), dtype=torch.float32, device=dev)
    pl = torch.full((S, wl.hq), float("nan"), dtype=torch.float32, device=dev)
    po = torch.full((S, wl.hq, wl.head_dim), float("nan"), dtype=torch.float32, device=dev)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=dev)
    if fp8:
        lb.attn_splitkv_fp8(q, kc, vc, inputs[4], inputs[5], bt, lens, mp, hdr["W"], hdr["S"], G, SCALE, pm, pl, po)
    else:
        lb.attn_splitkv(q, kc, vc, bt, lens, mp, hdr["W"], hdr["S"], G, SCALE, pm, pl, po)
    lb.attn_combine(pm, pl, po, mp, hdr["U"], out, max_splits=lb.max_splits_of(words))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"{what} request {b} (L={wl.kv_lens[b]})")


@pytest.mark.parametrize("seed", range(32))
def test_prefill_sweep(seed):
    from load_balanced_split_attn_amd.prefill import PrefillStep
    g = _rng(2, seed)
    batch = int(g.integers(1, 5))
    max_prefix = int(g.choice([0, 500, 2000]))
    max_chunk = int(g.integers(1, 401))
    wl = WL.random_prefill(700 + seed, batch, max_prefix, max_chunk)
    W = int(g.integers(1, 21))
    q_tile = int(g.choice([128, 256]))
    kv_tile = int(g.choice([64, 256, 512]))
    page = int(g.choice([64, 128]))
    exact_pv = [None, True, False][int(g.integers(0, 3))]
    causal = bool(g.random() < 0.75)
    note(f"prefill sweep {seed}: q={wl.q_lens} kv={wl.kv_lens} W={W} q_tile={q_tile} kv_tile={kv_tile} "
         f"page={page} exact_pv={exact_pv} causal={causal}")
    q, kc, vc, bt = prefill_inputs(wl, page=page, pad_value=float("nan"))
    step = PrefillStep(wl.q_lens, wl.kv_lens, q.device, num_workers=W, kv_tile=kv_tile, causal=causal,
                       exact_pv=exact_pv, q_tile=q_tile)
    assert np.array_equal(step.map_host, ref_plan_prefill(wl.q_lens, wl.kv_lens, W, q_tile, kv_tile, causal))
    for t in (step.part_m, step.part_l, step.part_o):
        t.fill_(float("nan"))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    starts = q_starts(wl)
    for b in range(wl.batch):
        k, v = wl.kv(b)
        ref = ref_attention(wl.q(b).double().numpy(), k.double().numpy(), v.double().numpy(), SCALE, causal=causal)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"prefill sweep {seed} request {b}")


@pytest.mark.parametrize("seed", range(32))
def test_mtp_sweep(lb, seed):
    from load_balanced_split_attn_amd.mtp import MtpDecodeStep
    g = _rng(3, seed)
    batch = int(g.integers(1, 9))
    wl = WL.random_mtp(800 + seed, batch, int(g.choice([300, 2000, 5000])))
    W = int(g.integers(1, 31))
    tile = int(g.choice([64, 256, 512]))
    page = int(g.choice([64, 128, 256]))
    fp8 = bool(g.random() < 0.5)
    note(f"mtp sweep {seed}: kv={wl.kv_lens} q={wl.q_lens} W={W} tile={tile} page={page} fp8={fp8}")
    q, kc, vc, bt, scales = mtp_inputs(wl, page=page, fp8=fp8, pad=NAN_CODE if fp8 else float("nan"))
    step = MtpDecodeStep(wl.q_lens, wl.kv_lens, q.device, num_workers=W, tile=tile, head_groups=8,
                         kv_dtype=lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16)
    assert np.array_equal(step.map_host, ref_plan_prefill(wl.q_lens, wl.kv_lens, W, step.R, tile, True))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out, kv_scales=scales)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    starts = q_starts(wl)
    for b, r in oracle_mtp(wl, fp8=fp8).items():
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], r, f"mtp sweep {seed} request {b}")
