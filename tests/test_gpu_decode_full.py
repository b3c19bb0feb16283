"""Full-size decode workloads in the launch configuration bench.py times (workers from the device
occupancy query, 512-token tiles, one workgroup per KV head, the launch order the step picks:
list-major for the balanced mixed and uniform batches): every request against the fp64
oracle, and all requests against the static split-KV map (an exact re-association, so the two must agree to fp32
rounding)."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import SCALE, assert_close, decode_inputs, errors, note, oracle_decode

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["uniform", "mixed", "long_tail", "control"])
def test_full_size(name):
    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.decode import DecodeStep
    from oracle.plan import ref_plan
    wl = WL.BY_NAME[name]()
    note(f"full-size {name}: B={wl.batch} tokens={sum(wl.kv_lens)}")
    q, kc, vc, bt = decode_inputs(wl)
    W = lb.attn_query_workers(0, 8)
    step = DecodeStep(wl.kv_lens, q.device, num_workers=W, head_groups=8)
    assert np.array_equal(step.map_host, ref_plan(wl.kv_lens, W, 512))
    note(f"  W={W}, launch order {'list' if step.list_major else 'head'}-major")
    out = step(q, kc, vc, bt, scale=SCALE)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    # every request against the fp64 oracle, one request at a time
    worst = (0.0, 0.0)
    for b in range(wl.batch):
        ma, rr = assert_close(got[b], oracle_decode(wl, [b])[b], f"{name} request {b} (L={wl.kv_lens[b]})")
        worst = (max(worst[0], ma), max(worst[1], rr))
    note(f"  all {wl.batch} requests: worst max_abs={worst[0]:.2e} rel_rms={worst[1]:.2e}")
    # every request: static split-KV map gives the same attention
    plain = min(max(1, -(-W // wl.batch)), max(-(-L // 512) for L in wl.kv_lens))
    st = DecodeStep(wl.kv_lens, q.device, head_groups=8, static_splits=plain)
    out2 = st(q, kc, vc, bt, scale=SCALE)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        assert errors(out2[b].cpu().numpy().astype(np.float64), got[b].astype(np.float64))[1] <= 1e-5


@pytest.mark.parametrize("name", ["mixed", "long_tail"])
def test_full_size_fp8(name):
    """The 8-bit cache path at full size, workers from the occupancy query of its own kernel; every
    request against the oracle."""
    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.decode import DecodeStep
    from gpu_helpers import decode_inputs_fp8, oracle_decode_fp8
    wl = WL.BY_NAME[name]()
    note(f"full-size fp8 {name}: B={wl.batch} tokens={sum(wl.kv_lens)}")
    q, kc, vc, bt, ks, vs = decode_inputs_fp8(wl)
    step = DecodeStep(wl.kv_lens, q.device, head_groups=8, kv_dtype=lb.KV_FP8_E4M3)
    out = step(q, kc, vc, bt, scale=SCALE, kv_scales=(ks, vs))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    worst = (0.0, 0.0)
    for b in range(wl.batch):
        ma, rr = assert_close(got[b], oracle_decode_fp8(wl, [b])[b], f"fp8 {name} request {b} (L={wl.kv_lens[b]})")
        worst = (max(worst[0], ma), max(worst[1], rr))
    note(f"  all {wl.batch} requests: worst max_abs={worst[0]:.2e} rel_rms={worst[1]:.2e}")


@pytest.mark.parametrize("fp8", [False, True])
def test_full_size_kv_head_share(fp8):
    """One GPU's share of the mixed batch under 8-way KV-head sharding (8 query heads over one KV
    head) in the launch bench.py times: 1,024 workers, one wave per (worker, KV head); every request
    against the fp64 oracle and against the plain static split map."""
    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.decode import DecodeStep
    from gpu_helpers import decode_inputs_fp8, oracle_decode_fp8
    from oracle.plan import ref_plan
    wl = WL.BY_NAME["mixed_tp8"]()
    assert (wl.hq, wl.hkv) == (8, 1)
    note(f"full-size KV-head share ({'E4M3' if fp8 else 'bf16'}): B={wl.batch} tokens={sum(wl.kv_lens)}")
    kw = dict(num_q_heads=wl.hq, head_groups=1)
    if fp8:
        q, kc, vc, bt, ks, vs = decode_inputs_fp8(wl)
        kw["kv_dtype"] = lb.KV_FP8_E4M3
        call = dict(kv_scales=(ks, vs))
    else:
        q, kc, vc, bt = decode_inputs(wl)
        call = {}
    step = DecodeStep(wl.kv_lens, q.device, num_workers=1024, **kw)
    assert np.array_equal(step.map_host, ref_plan(wl.kv_lens, 1024, 512))
    out = step(q, kc, vc, bt, scale=SCALE, **call)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    oracle = oracle_decode_fp8 if fp8 else oracle_decode
    worst = (0.0, 0.0)
    for b in range(wl.batch):
        ma, rr = assert_close(got[b], oracle(wl, [b])[b], f"share request {b} (L={wl.kv_lens[b]})")
        worst = (max(worst[0], ma), max(worst[1], rr))
    note(f"  all {wl.batch} requests: worst max_abs={worst[0]:.2e} rel_rms={worst[1]:.2e}")
    st = DecodeStep(wl.kv_lens, q.device, static_splits=26, **kw)
    out2 = st(q, kc, vc, bt, scale=SCALE, **call)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        assert errors(out2[b].cpu().numpy().astype(np.float64), got[b].astype(np.float64))[1] <= 1e-5


def test_full_size_million_token_request():
    """Maximum-size case: one request of 2^20 tokens (16,384 pages, so cache offsets pass 2^31
    bytes) beside three short ones, in the launch bench.py times (workers from the occupancy query,
    512-token tiles, one wave per KV head).  The long request is cut over every worker and its
    ~128 splits take the many-split combine; every request is checked against the fp64 oracle."""
    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.decode import DecodeStep
    from oracle.plan import ref_plan
    wl = WL.random_decode(21, 4, 3000, min_len=1)
    wl.kv_lens[1] = 1 << 20
    note(f"million-token request: lengths {wl.kv_lens}")
    q, kc, vc, bt = decode_inputs(wl)
    assert kc.numel() * kc.element_size() > 2 ** 31
    W = lb.attn_query_workers(0, 8)
    step = DecodeStep(wl.kv_lens, q.device, num_workers=W, head_groups=8)
    assert np.array_equal(step.map_host, ref_plan(wl.kv_lens, W, 512))
    assert step.max_splits > 16
    out = step(q, kc, vc, bt, scale=SCALE)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del kc, vc
    torch.cuda.empty_cache()
    for b in range(wl.batch):
        ref = oracle_decode(wl, [b])[b]
        ma, rr = assert_close(got[b], ref, f"request {b} (L={wl.kv_lens[b]})")
        note(f"  request {b} L={wl.kv_lens[b]}: max_abs={ma:.2e} rel_rms={rr:.2e}")
