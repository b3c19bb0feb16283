"""GPU parity of the decode path (attn_plan -> attn_splitkv -> attn_combine through the C ABI)
against the fp64 oracle, on small seeded batches that span several tiles and ragged tails."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import SCALE, assert_close, decode_inputs, errors, note, oracle_decode
from oracle.attention import ref_split_partials
from oracle.plan import ref_plan, ref_plan_static

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _run(lb, wl, words, head_groups=8, pad_value=0.0, out_dtype=torch.float32, poison=False, inputs=None):
    from load_balanced_split_attn_amd import map_header
    q, kc, vc, bt = inputs if inputs is not None else decode_inputs(wl, pad_value=pad_value)
    hdr = map_header(words)
    dev = q.device
    mp = torch.from_numpy(np.asarray(words, dtype=np.int32)).to(dev)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    S = max(hdr["S"], 1)
    fill = float("nan") if poison else 0.0
    pm = torch.full((S, wl.hq), fill, dtype=torch.float32, device=dev)
    pl = torch.full((S, wl.hq), fill, dtype=torch.float32, device=dev)
    po = torch.full((S, wl.hq, wl.head_dim), fill, dtype=torch.float32, device=dev)
    out = torch.full(q.shape, fill, dtype=out_dtype, device=dev)
    lb.attn_splitkv(q, kc, vc, bt, lens, mp, hdr["W"], hdr["S"], head_groups, SCALE, pm, pl, po)
    lb.attn_combine(pm, pl, po, mp, hdr["U"], out)
    torch.cuda.synchronize()
    return out, (pm, pl, po)


def test_tiny_worked_example(lb):
    wl = WL.tiny()
    words = lb.attn_plan(wl.kv_lens, 4, 512)
    assert np.array_equal(words, ref_plan(wl.kv_lens, 4, 512))
    ref = oracle_decode(wl)
    for G in (8, 1):
        note(f"tiny worked example, head_groups={G}")
        out, parts = _run(lb, wl, words, head_groups=G)
        got = out.cpu().numpy()
        for b in range(wl.batch):
            assert_close(got[b], ref[b], f"request {b} G={G}")
    # partial-level diagnostics against the oracle's per-split partials
    q = wl.q().double().numpy()
    kvs = [wl.kv(b) for b in range(wl.batch)]
    rparts = ref_split_partials(words, [q[b:b + 1] for b in range(wl.batch)],
                                [k.double().numpy() for k, _ in kvs], [v.double().numpy() for _, v in kvs], SCALE)
    pm, pl, po = (t.cpu().numpy() for t in parts)
    for s, (m, l, o) in enumerate(rparts):
        assert np.max(np.abs(pm[s] - m[0])) <= 1e-3, f"slot {s} m"
        lse_got = pm[s] + np.log(pl[s])
        lse_ref = m[0] + np.log(l[0])
        assert np.max(np.abs(lse_got - lse_ref)) <= 1e-3, f"slot {s} lse"
        assert_close(po[s] / pl[s][:, None], o[0] / l[0][:, None], f"slot {s} o/l")


@pytest.mark.parametrize("seed,batch,max_len,W,G", [
    (0, 6, 3000, 7, 8), (1, 9, 1500, 1, 8), (2, 5, 5000, 64, 4), (3, 12, 700, 100, 2),
    (4, 4, 2600, 3, 1), (5, 7, 1100, 2000, 8),
])
def test_random_ragged(lb, seed, batch, max_len, W, G):
    wl = WL.random_decode(seed, batch, max_len)
    wl.kv_lens[0] = 0                           # an empty request
    wl.kv_lens[-1] = max(wl.kv_lens[-1], 513)   # a ragged tail past one tile
    note(f"random ragged seed={seed} lens={wl.kv_lens} W={W} G={G}")
    words = lb.attn_plan(wl.kv_lens, W, 512)
    assert np.array_equal(words, ref_plan(wl.kv_lens, W, 512))
    out, _ = _run(lb, wl, words, head_groups=G, pad_value=float("nan"), poison=True)
    got = out.cpu().numpy()
    ref = oracle_decode(wl)
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"seed {seed} request {b} (L={wl.kv_lens[b]})")


def test_maps_agree_and_paging_invariance(lb):
    wl = WL.random_decode(11, 8, 4000, min_len=1)
    note(f"map agreement lens={wl.kv_lens}")
    inputs = decode_inputs(wl)
    outs = []
    for words in (lb.attn_plan(wl.kv_lens, 37, 512), lb.attn_plan(wl.kv_lens, 1, 512),
                  lb.attn_plan_static(wl.kv_lens, 1, 512), lb.attn_plan_static(wl.kv_lens, 3, 512),
                  lb.attn_plan(wl.kv_lens, 37, 64), lb.attn_plan_lpt(wl.kv_lens, 37, 512),
                  lb.attn_plan_lpt(wl.kv_lens, 5, 64)):
        out, _ = _run(lb, wl, words, inputs=inputs)
        outs.append(out.cpu().numpy().astype(np.float64))
    for o in outs[1:]:
        assert errors(o, outs[0])[1] <= 1e-5
    # same map, two runs: bitwise equal
    words = lb.attn_plan(wl.kv_lens, 37, 512)
    a, _ = _run(lb, wl, words, inputs=inputs)
    b, _ = _run(lb, wl, words, inputs=inputs)
    assert torch.equal(a, b)
    # a different physical page order gives bitwise the same result
    wl2 = WL.random_decode(11, 8, 4000, min_len=1)
    wl2.page_permutation = lambda n: torch.randperm(n, generator=torch.Generator().manual_seed(99))
    c, _ = _run(lb, wl2, words)
    assert torch.equal(a, c)


def test_combine_many_splits(lb):
    """A long request cut over many workers: the four-waves-per-unit combine (max_splits > 16) and
    the one-wave combine agree, and both match the oracle."""
    wl = WL.random_decode(14, 3, 100, min_len=50)
    wl.kv_lens[1] = 40000          # 79 tiles of 512 over 120 workers -> many one-tile splits
    words = lb.attn_plan(wl.kv_lens, 120, 512)
    assert lb.max_splits_of(words) > 16
    inputs = decode_inputs(wl)
    from load_balanced_split_attn_amd import map_header
    hdr = map_header(words)
    q = inputs[0]
    mp = torch.from_numpy(words).to(q.device)
    _, (pm, pl, po) = _run(lb, wl, words, inputs=inputs)
    outs = []
    for ms in (0, lb.max_splits_of(words)):
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
        lb.attn_combine(pm, pl, po, mp, hdr["U"], out, max_splits=ms)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert errors(outs[0].astype(np.float64), outs[1].astype(np.float64))[1] <= 1e-6
    ref = oracle_decode(wl)
    for b in range(wl.batch):
        assert_close(outs[1][b], ref[b], f"many-split request {b}")


def test_bf16_output(lb):
    wl = WL.random_decode(12, 4, 2000, min_len=600)
    words = lb.attn_plan(wl.kv_lens, 16, 512)
    out, _ = _run(lb, wl, words, out_dtype=torch.bfloat16)
    ref = oracle_decode(wl)
    got = out.float().cpu().numpy()
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"bf16 request {b}")


def test_timing_records(lb):
    wl = WL.random_decode(13, 4, 3000, min_len=1000)
    q, kc, vc, bt = decode_inputs(wl)
    from load_balanced_split_attn_amd.decode import DecodeStep
    step = DecodeStep(wl.kv_lens, q.device, num_workers=20, head_groups=8)
    timing = torch.zeros((20 * 8, 4), dtype=torch.int64, device=q.device)
    out = step(q, kc, vc, bt, timing=timing)
    torch.cuda.synchronize()
    t = timing.cpu().numpy()
    assert np.all(t[:, 1] >= t[:, 0]) and np.all(t[:, 0] > 0)
    assert np.all((t[:, 3] & 0xF) < 8)
    ref = oracle_decode(wl)
    for b in range(wl.batch):
        assert_close(out[b].cpu().numpy(), ref[b], f"timed run request {b}")


@pytest.mark.parametrize("tile,split_cost", [(512, 0), (128, 128), (64, 300)])
def test_weighted_map_partials(lb, tile, split_cost):
    """A cost-weighted map (segments cut at any tile boundary, partial tiles weighted by their
    tokens): every slot's partial and the combined output match the oracle's."""
    wl = WL.random_decode(17 + tile, 7, 3000, min_len=1)
    words = lb.attn_plan_weighted(wl.kv_lens, 10, tile, split_cost)
    from oracle.plan import ref_plan_weighted
    assert np.array_equal(words, ref_plan_weighted(wl.kv_lens, 10, tile, split_cost))
    out, parts = _run(lb, wl, words, poison=True)
    ref = oracle_decode(wl)
    got = out.cpu().numpy()
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"weighted request {b}")
    q = wl.q().double().numpy()
    kvs = [wl.kv(b) for b in range(wl.batch)]
    rparts = ref_split_partials(words, [q[b:b + 1] for b in range(wl.batch)],
                                [k.double().numpy() for k, _ in kvs], [v.double().numpy() for _, v in kvs], SCALE)
    pm, pl, po = (t.cpu().numpy() for t in parts)
    for s_, (m, l, o) in enumerate(rparts):
        assert np.max(np.abs(pm[s_] - m[0])) <= 1e-3, f"slot {s_} m"
        assert_close(po[s_] / pl[s_][:, None], o[0] / l[0][:, None], f"slot {s_} o/l")


def test_lpt_map_partials(lb):
    """A version-2 (LPT) map: every slot's partial matches the oracle's partial of that segment, and
    the combined output matches the oracle."""
    wl = WL.random_decode(16, 5, 3000, min_len=300)
    words = lb.attn_plan_lpt(wl.kv_lens, 9, 512)
    from oracle.plan import ref_plan_lpt
    assert np.array_equal(words, ref_plan_lpt(wl.kv_lens, 9, 512))
    out, parts = _run(lb, wl, words, poison=True)
    ref = oracle_decode(wl)
    got = out.cpu().numpy()
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"lpt request {b}")
    q = wl.q().double().numpy()
    kvs = [wl.kv(b) for b in range(wl.batch)]
    rparts = ref_split_partials(words, [q[b:b + 1] for b in range(wl.batch)],
                                [k.double().numpy() for k, _ in kvs], [v.double().numpy() for _, v in kvs], SCALE)
    pm, pl, po = (t.cpu().numpy() for t in parts)
    for s_, (m, l, o) in enumerate(rparts):
        assert np.max(np.abs(pm[s_] - m[0])) <= 1e-3, f"slot {s_} m"
        assert_close(po[s_] / pl[s_][:, None], o[0] / l[0][:, None], f"slot {s_} o/l")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("launch_workers", [6, 4])
def test_worker_count_mismatch_writes_nothing(lb, launch_workers, fp8):
    """A map planned for five workers launched with another worker count is skipped on the device
    (its lists are never read past their end), for a larger and a smaller grid, both caches."""
    from gpu_helpers import decode_inputs_fp8
    wl = WL.random_decode(14, 6, 2000)
    words = lb.attn_plan(wl.kv_lens, 5, 512)
    inputs = decode_inputs_fp8(wl) if fp8 else decode_inputs(wl)
    q, kc, vc, bt = inputs[:4]
    dev = q.device
    mp = torch.from_numpy(np.asarray(words, dtype=np.int32)).to(dev)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    S = max(int(words[4]), 1)
    pm = torch.full((S, wl.hq), 7.0, device=dev)
    pl = torch.full((S, wl.hq), 7.0, device=dev)
    po = torch.full((S, wl.hq, wl.head_dim), 7.0, device=dev)
    if fp8:
        lb.attn_splitkv_fp8(q, kc, vc, inputs[4], inputs[5], bt, lens, mp, launch_workers, int(words[4]), 8, SCALE,
                            pm, pl, po)
    else:
        lb.attn_splitkv(q, kc, vc, bt, lens, mp, launch_workers, int(words[4]), 8, SCALE, pm, pl, po)
    torch.cuda.synchronize()
    assert bool((pm == 7.0).all()) and bool((pl == 7.0).all()) and bool((po == 7.0).all())


def test_two_streams_concurrently(lb):
    """The library keeps no per-call global state: two different decode batches launched on two
    streams at once (split-KV and combine interleaved on the device) give bitwise the results of
    running them one after the other."""
    from load_balanced_split_attn_amd.decode import DecodeStep
    wls = [WL.random_decode(31, 9, 9000, min_len=1), WL.random_decode(32, 5, 30000, min_len=500)]
    inputs = [decode_inputs(w) for w in wls]
    steps = [DecodeStep(w.kv_lens, inp[0].device, num_workers=W) for w, inp, W in zip(wls, inputs, (37, 64))]
    seq = []
    for st, (q, kc, vc, bt) in zip(steps, inputs):
        seq.append(st(q, kc, vc, bt, scale=SCALE).clone())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    outs = [torch.full(inp[0].shape, float("nan"), dtype=torch.float32, device=inp[0].device) for inp in inputs]
    torch.cuda.synchronize()
    for rep in range(3):
        for st, (q, kc, vc, bt), s, o in zip(steps, inputs, streams, outs):
            st.splitkv(q, kc, vc, bt, SCALE, stream=s)
        for st, s, o in zip(steps, streams, outs):
            st.combine(o, stream=s)
        torch.cuda.synchronize()
        for a, b in zip(seq, outs):
            assert torch.equal(a, b)
    ref = oracle_decode(wls[1], [0, 4])
    for b, r in ref.items():
        assert_close(outs[1][b].cpu().numpy(), r, f"stream request {b}")
