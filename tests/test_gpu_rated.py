"""Version-3 maps (attn_plan_rated) through the C ABI: the split-KV launch runs workgroup b on list
b mod W and head group b div W.

* Equal rates give attn_plan_weighted's lists, so every partial and the combined output must be
  bitwise those of the head-major launch over the weighted version-1 map (head groups 8, 4, 2, 1;
  W a multiple of 8 or not): the list-major order covers every (list, head group) exactly once.
* Uneven rates (zeros included, tiles of 128 and 512, a split cost): every slot's partial and the
  output against the fp64 oracle, bf16 and E4M3 caches.
* Calibrated: per-XCD rates from the kernel's own timestamps on the mixed batch, then the rated step
  at full size against the default step (an exact re-association: rel-RMS 1e-5) and the oracle on a
  sample of requests.
* Launch order of a version-1 map (DecodeStep's launch_order): head-major and list-major give the
  same partials bit for bit, and "auto" picks list-major only where the per-XCD totals are balanced.
"""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import (SCALE, assert_close, decode_inputs, decode_inputs_fp8, errors, note, oracle_decode,
                         oracle_decode_fp8)
from oracle.attention import ref_split_partials
from oracle.plan import ref_plan_rated

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _run(lb, wl, words, G, inputs, fp8=False):
    q, kc, vc, bt = inputs[:4]
    hdr = lb.map_header(words)
    dev = q.device
    mp = torch.from_numpy(np.asarray(words, dtype=np.int32)).to(dev)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    S = max(hdr["S"], 1)
    pm = torch.full((S, wl.hq), float("nan"), device=dev)
    pl = torch.full((S, wl.hq), float("nan"), device=dev)
    po = torch.full((S, wl.hq, wl.head_dim), float("nan"), device=dev)
    out = torch.full(q.shape, float("nan"), device=dev)
    if fp8:
        lb.attn_splitkv_fp8(q, kc, vc, inputs[4], inputs[5], bt, lens, mp, hdr["W"], hdr["S"], G, SCALE, pm, pl, po)
    else:
        lb.attn_splitkv(q, kc, vc, bt, lens, mp, hdr["W"], hdr["S"], G, SCALE, pm, pl, po)
    lb.attn_combine(pm, pl, po, mp, hdr["U"], out)
    torch.cuda.synchronize()
    return out, (pm, pl, po)


@pytest.mark.parametrize("G", [8, 4, 2, 1])
@pytest.mark.parametrize("W,tile,split_cost", [(16, 512, 0), (10, 128, 64), (24, 64, 0)])
def test_equal_rates_bitwise_as_weighted(lb, G, W, tile, split_cost):
    wl = WL.random_decode(40 + W + G, 9, 4000, min_len=0)
    note(f"rated equal rates G={G} W={W} tile={tile} split_cost={split_cost}")
    inputs = decode_inputs(wl)
    rated = lb.attn_plan_rated(wl.kv_lens, W, [7] * W, tile, split_cost)
    weighted = lb.attn_plan_weighted(wl.kv_lens, W, tile, split_cost)
    assert rated[0] == 3 and weighted[0] == 1 and np.array_equal(rated[1:], weighted[1:])
    out_r, parts_r = _run(lb, wl, rated, G, inputs)
    out_w, parts_w = _run(lb, wl, weighted, G, inputs)
    for a, b in zip(parts_r, parts_w):
        assert torch.equal(a.nan_to_num(123.0), b.nan_to_num(123.0))
    assert torch.equal(out_r, out_w)
    assert torch.isfinite(out_r).all()


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("tile,split_cost,rates", [
    (512, 0, [65536, 61000, 65536, 60000, 64000, 0, 65000, 62000, 1, 65536]),
    (128, 128, [3, 1, 0, 0, 5, 2, 2, 9, 4, 1]),
])
def test_uneven_rates_against_oracle(lb, fp8, tile, split_cost, rates):
    wl = WL.random_decode(77 + tile, 8, 6000, min_len=1)
    W = len(rates)
    note(f"rated uneven rates fp8={fp8} tile={tile} split_cost={split_cost}")
    words = lb.attn_plan_rated(wl.kv_lens, W, rates, tile, split_cost)
    assert np.array_equal(words, ref_plan_rated(wl.kv_lens, W, tile, split_cost, rates))
    inputs = decode_inputs_fp8(wl) if fp8 else decode_inputs(wl)
    out, parts = _run(lb, wl, words, 8, inputs, fp8=fp8)
    got = out.cpu().numpy()
    ref = oracle_decode_fp8(wl) if fp8 else oracle_decode(wl)
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"rated request {b}")
    if not fp8:
        q = wl.q().double().numpy()
        kvs = [wl.kv(b) for b in range(wl.batch)]
        rparts = ref_split_partials(words, [q[b:b + 1] for b in range(wl.batch)],
                                    [k.double().numpy() for k, _ in kvs], [v.double().numpy() for _, v in kvs], SCALE)
        pm, pl, po = (t.cpu().numpy() for t in parts)
        for s_, (m, l, o) in enumerate(rparts):
            assert np.max(np.abs(pm[s_] - m[0])) <= 1e-3, f"slot {s_} m"
            assert_close(po[s_] / pl[s_][:, None], o[0] / l[0][:, None], f"slot {s_} o/l")


def test_calibrated_rates_full_size_mixed(lb):
    from load_balanced_split_attn_amd.decode import DecodeStep, calibrate_xcd_rates
    wl = WL.mixed()
    note(f"rated calibrated: mixed B={wl.batch}")
    q, kc, vc, bt = decode_inputs(wl)
    base = DecodeStep(wl.kv_lens, q.device, head_groups=8)
    rates = calibrate_xcd_rates(base, q, kc, vc, bt, SCALE)
    note(f"  per-XCD rates {rates}")
    assert len(rates) == 8 and max(rates) == 1 << 16 and min(rates) >= (1 << 16) // 2
    W = base.W
    step = DecodeStep(wl.kv_lens, q.device, num_workers=W, head_groups=8, planner="rated", xcd_rates=rates)
    assert np.array_equal(step.map_host, ref_plan_rated(wl.kv_lens, W, 512, 0, [rates[w % 8] for w in range(W)]))
    ref_out = base(q, kc, vc, bt, scale=SCALE)
    out = step(q, kc, vc, bt, scale=SCALE)
    torch.cuda.synchronize()
    got, want = out.cpu().numpy().astype(np.float64), ref_out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    for b in range(wl.batch):
        assert errors(got[b], want[b])[1] <= 1e-5, f"request {b}"
    for b in (0, 7, 21, 39):
        assert_close(got[b], oracle_decode(wl, [b])[b], f"rated mixed request {b} (L={wl.kv_lens[b]})")


@pytest.mark.parametrize("G", [8, 4, 2])
def test_launch_order_bitwise(lb, G):
    """A version-1 map launched head-major and list-major (its device word 0 set to 3): the same
    partials and output bit for bit; the host map stays the oracle's."""
    from load_balanced_split_attn_amd.decode import DecodeStep
    from oracle.plan import ref_plan
    wl = WL.random_decode(123 + G, 11, 7000, min_len=1)
    q, kc, vc, bt = decode_inputs(wl)
    note(f"launch order G={G}")
    outs, parts = [], []
    for order in ("head", "list"):
        st = DecodeStep(wl.kv_lens, q.device, num_workers=16, head_groups=G, launch_order=order)
        assert np.array_equal(st.map_host, ref_plan(wl.kv_lens, 16, 512))
        assert st.list_major == (order == "list")
        assert int(st.map[0].item()) == (3 if order == "list" else 1)
        for t in (st.part_m, st.part_l, st.part_o):
            t.fill_(float("nan"))
        outs.append(st(q, kc, vc, bt, scale=SCALE))
        parts.append([t.clone() for t in (st.part_m, st.part_l, st.part_o)])
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    for a, b in zip(*parts):
        assert torch.equal(a, b)


def test_launch_order_auto_choice(lb):
    """"auto" launches list-major where the per-XCD token totals under it are within 1% (the mixed
    batch) and head-major where they are not (the long-tail batch), at the device's worker count."""
    from load_balanced_split_attn_amd.decode import DecodeStep
    mixed = DecodeStep(WL.mixed().kv_lens, "cuda", head_groups=8)
    tail = DecodeStep(WL.long_tail().kv_lens, "cuda", head_groups=8)
    note(f"auto order: mixed W={mixed.W} list-major={mixed.list_major}, long tail W={tail.W} "
         f"list-major={tail.list_major}")
    if mixed.W % 8 == 0:
        assert mixed.list_major and int(mixed.map[0].item()) == 3 and int(mixed.map_host[0]) == 1
    assert not tail.list_major and int(tail.map[0].item()) == 1
