"""Full-size decode workloads in the launch configuration bench.py times (workers from the device
occupancy query, 512-token tiles, one workgroup per KV head): sampled requests against the fp64
oracle, and all requests against the static split-KV map (an exact re-association, so the two must
agree to fp32 rounding)."""

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
    out = step(q, kc, vc, bt, scale=SCALE)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    # sampled requests: one of each distinct length (the longest included) and the first two
    seen, sample = set(), [0, 1]
    for b, L in enumerate(wl.kv_lens):
        if L not in seen:
            seen.add(L)
            sample.append(b)
    sample = sorted(set(sample))[:8] + [int(np.argmax(wl.kv_lens))]
    ref = oracle_decode(wl, sorted(set(sample)))
    for b, r in ref.items():
        ma, rr = assert_close(got[b], r, f"{name} request {b} (L={wl.kv_lens[b]})")
        note(f"  request {b} L={wl.kv_lens[b]}: max_abs={ma:.2e} rel_rms={rr:.2e}")
    # every request: static split-KV map gives the same attention
    plain = min(max(1, -(-W // wl.batch)), max(-(-L // 512) for L in wl.kv_lens))
    st = DecodeStep(wl.kv_lens, q.device, head_groups=8, static_splits=plain)
    out2 = st(q, kc, vc, bt, scale=SCALE)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        assert errors(out2[b].cpu().numpy().astype(np.float64), got[b].astype(np.float64))[1] <= 1e-5


@pytest.mark.parametrize("name", ["mixed", "long_tail"])
def test_full_size_fp8(name):
    """The 8-bit cache path at full size, workers from the occupancy query of its own kernel."""
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
    seen, sample = set(), [0]
    for b, L in enumerate(wl.kv_lens):
        if L not in seen:
            seen.add(L)
            sample.append(b)
    sample = sorted(set(sample[:6] + [int(np.argmax(wl.kv_lens))]))
    ref = oracle_decode_fp8(wl, sample)
    for b, r in ref.items():
        ma, rr = assert_close(got[b], r, f"fp8 {name} request {b} (L={wl.kv_lens[b]})")
        note(f"  request {b} L={wl.kv_lens[b]}: max_abs={ma:.2e} rel_rms={rr:.2e}")
