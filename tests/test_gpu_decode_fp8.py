"""GPU parity of the decode path over an 8-bit (E4M3) KV cache with per-head scales
(attn_plan -> attn_splitkv_fp8 -> attn_combine through the C ABI) against the fp64 oracle, which
dequantises the same codes and runs plain attention."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import SCALE, assert_close, decode_inputs_fp8, errors, note, oracle_decode_fp8
from oracle.fp8 import dequantize_kv, e4m3_table
from oracle.attention import ref_split_partials
from oracle.plan import ref_plan, ref_plan_static

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _run(lb, wl, words, inputs, head_groups=8, poison=False):
    from load_balanced_split_attn_amd import map_header
    q, kc, vc, bt, ks, vs = inputs
    hdr = map_header(words)
    dev = q.device
    mp = torch.from_numpy(np.asarray(words, dtype=np.int32)).to(dev)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    S = max(hdr["S"], 1)
    fill = float("nan") if poison else 0.0
    pm = torch.full((S, wl.hq), fill, dtype=torch.float32, device=dev)
    pl = torch.full((S, wl.hq), fill, dtype=torch.float32, device=dev)
    po = torch.full((S, wl.hq, wl.head_dim), fill, dtype=torch.float32, device=dev)
    out = torch.full(q.shape, fill, dtype=torch.float32, device=dev)
    lb.attn_splitkv_fp8(q, kc, vc, ks, vs, bt, lens, mp, hdr["W"], hdr["S"], head_groups, SCALE, pm, pl, po)
    lb.attn_combine(pm, pl, po, mp, hdr["U"], out, max_splits=lb.max_splits_of(words))
    torch.cuda.synchronize()
    return out, (pm, pl, po)


def test_tiny_worked_example_fp8(lb):
    wl = WL.tiny()
    words = lb.attn_plan(wl.kv_lens, 4, 512)
    inputs = decode_inputs_fp8(wl)
    ref = oracle_decode_fp8(wl)
    for G in (8, 1):
        note(f"fp8 tiny worked example, head_groups={G}")
        out, parts = _run(lb, wl, words, inputs, head_groups=G)
        got = out.cpu().numpy()
        for b in range(wl.batch):
            ma, rr = assert_close(got[b], ref[b], f"fp8 request {b} G={G}")
            note(f"  request {b}: max_abs={ma:.2e} rel_rms={rr:.2e}")
    # partial-level diagnostics against the oracle's per-split partials of the dequantised cache
    q = wl.q().double().numpy()
    ks, vs = (s.double().numpy() for s in wl.kv_scales())
    kd, vd = [], []
    for b in range(wl.batch):
        k, v = wl.kv_fp8(b)
        kd.append(dequantize_kv(k.numpy(), ks))
        vd.append(dequantize_kv(v.numpy(), vs))
    rparts = ref_split_partials(words, [q[b:b + 1] for b in range(wl.batch)], kd, vd, SCALE)
    pm, pl, po = (t.cpu().numpy() for t in parts)
    for s, (m, l, o) in enumerate(rparts):
        assert np.max(np.abs(pm[s] - m[0])) <= 1e-3, f"slot {s} m"
        assert np.max(np.abs(pm[s] + np.log(pl[s]) - (m[0] + np.log(l[0])))) <= 1e-3, f"slot {s} lse"
        assert_close(po[s] / pl[s][:, None], o[0] / l[0][:, None], f"slot {s} o/l")


@pytest.mark.parametrize("seed,batch,max_len,W,G", [
    (0, 6, 3000, 7, 8), (1, 9, 1500, 1, 8), (2, 5, 5000, 64, 4), (3, 12, 700, 100, 2),
    (4, 4, 2600, 3, 1), (5, 7, 1100, 2000, 8),
])
def test_random_ragged_fp8(lb, seed, batch, max_len, W, G):
    wl = WL.random_decode(seed, batch, max_len)
    wl.kv_lens[0] = 0                           # an empty request
    wl.kv_lens[-1] = max(wl.kv_lens[-1], 513)   # a ragged tail past one tile
    note(f"fp8 random ragged seed={seed} lens={wl.kv_lens} W={W} G={G}")
    words = lb.attn_plan(wl.kv_lens, W, 512)
    assert np.array_equal(words, ref_plan(wl.kv_lens, W, 512))
    # tokens past a request's end hold NaN codes: they must not leak into the result
    out, _ = _run(lb, wl, words, decode_inputs_fp8(wl, pad_code=NAN_CODE), head_groups=G, poison=True)
    got = out.cpu().numpy()
    ref = oracle_decode_fp8(wl)
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"fp8 seed {seed} request {b} (L={wl.kv_lens[b]})")


def test_every_code_widens_exactly(lb):
    """One-key requests: each query head sees a single key, so its partial max is scale * k_scale *
    e4m3(code) for the key element its one-hot query picks, and the output is v_scale * e4m3(code)
    for every V element.  Together the requests cover all 254 finite codes in K and in V."""
    dev = torch.device("cuda")
    B, Hq, Hkv, D = 4, 64, 8, 128
    wl = WL.Workload("codes", 900, [1] * B, [1] * B, paged=False)
    table = e4m3_table()
    finite = np.isfinite(table)
    kcodes, vcodes = [], []
    for b in range(B):
        k = np.zeros((1, Hkv, D), dtype=np.uint8)
        for g in range(Hkv):
            for i in range(8):
                k[0, g, i] = (b * 64 + g * 8 + i) & 0xFF      # head 8g + i reads dim i
        v = (np.arange(Hkv * D, dtype=np.int64).reshape(1, Hkv, D) + b * 37) % 256
        v = v.astype(np.uint8)
        for a in (k, v):
            a[~finite[a]] = 0
        kcodes.append(torch.from_numpy(k))
        vcodes.append(torch.from_numpy(v))
    wl.kv_fp8 = lambda b: (kcodes[b], vcodes[b])
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16)
    for h in range(Hq):
        q[:, h, h % 8] = 1.0
    wl.q = lambda b=None: q
    inputs = decode_inputs_fp8(wl)
    words = lb.attn_plan(wl.kv_lens, 4, 512)
    out, (pm, pl, po) = _run(lb, wl, words, inputs)
    ks, vs = (s.double().numpy() for s in wl.kv_scales())
    pm, got = pm.cpu().numpy(), out.cpu().numpy()
    for b in range(B):
        exp_m = np.array([SCALE * ks[h // 8] * table[kcodes[b][0, h // 8, h % 8]] for h in range(Hq)])
        assert np.allclose(pm[b], exp_m, rtol=1e-6, atol=1e-30), f"request {b} partial max"
        exp_o = table[vcodes[b][0].numpy()] * vs[:, None]                        # [Hkv, D]
        assert np.allclose(got[b], np.repeat(exp_o, 8, axis=0), rtol=1e-6, atol=1e-30), f"request {b} output"
    k_seen = {int(kcodes[b][0, g, i]) for b in range(B) for g in range(Hkv) for i in range(8)}
    v_seen = {int(c) for b in range(B) for c in vcodes[b].flatten()}
    assert k_seen == v_seen == {c for c in range(256) if finite[c]}


def test_maps_agree_and_determinism_fp8(lb):
    wl = WL.random_decode(11, 8, 4000, min_len=1)
    inputs = decode_inputs_fp8(wl)
    outs = []
    for words in (lb.attn_plan(wl.kv_lens, 37, 512), lb.attn_plan(wl.kv_lens, 1, 512),
                  lb.attn_plan_static(wl.kv_lens, 3, 512), lb.attn_plan(wl.kv_lens, 37, 64)):
        out, _ = _run(lb, wl, words, inputs)
        outs.append(out.cpu().numpy().astype(np.float64))
    for o in outs[1:]:
        assert errors(o, outs[0])[1] <= 1e-5
    words = lb.attn_plan(wl.kv_lens, 37, 512)
    a, _ = _run(lb, wl, words, inputs)
    b, _ = _run(lb, wl, words, inputs)
    assert torch.equal(a, b)


def test_decode_step_fp8(lb):
    from load_balanced_split_attn_amd import KV_FP8_E4M3
    from load_balanced_split_attn_amd.decode import DecodeStep
    wl = WL.random_decode(15, 5, 3000, min_len=700)
    q, kc, vc, bt, ks, vs = decode_inputs_fp8(wl)
    step = DecodeStep(wl.kv_lens, q.device, head_groups=8, kv_dtype=KV_FP8_E4M3)
    assert step.W == lb.attn_query_workers(0, 8, KV_FP8_E4M3)
    out = step(q, kc, vc, bt, kv_scales=(ks, vs))
    torch.cuda.synchronize()
    ref = oracle_decode_fp8(wl)
    for b in range(wl.batch):
        assert_close(out[b].cpu().numpy(), ref[b], f"DecodeStep fp8 request {b}")
