"""Run-time claiming of the work map's lists (attn_splitkv_claimed): resident one-wave workgroups
take (list, KV head) items from a device counter.  Every item runs once and writes the slots the
static launch writes, so partials and outputs must equal the static launch's bit for bit, launch
after launch (the kernel leaves its counter state at zero), and match the fp64 oracle."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import (SCALE, assert_close, decode_inputs, decode_inputs_fp8, note, oracle_decode,
                         oracle_decode_fp8)
from oracle.plan import ref_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _compare(lb, wl, W, tile, resident, fp8, launches=3, oracle_requests=None):
    from load_balanced_split_attn_amd.decode import DecodeStep
    kvd = lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16
    if fp8:
        q, kc, vc, bt, ks, vs = decode_inputs_fp8(wl)
        scales = (ks, vs)
    else:
        q, kc, vc, bt = decode_inputs(wl)
        scales = None
    static = DecodeStep(wl.kv_lens, q.device, num_workers=W, tile=tile, head_groups=wl.hkv, num_q_heads=wl.hq,
                        kv_dtype=kvd)
    claimed = DecodeStep(wl.kv_lens, q.device, num_workers=W, tile=tile, head_groups=wl.hkv, num_q_heads=wl.hq,
                         kv_dtype=kvd, resident_workgroups=resident)
    assert np.array_equal(static.map_host, ref_plan(wl.kv_lens, W, tile))
    ref_out = static(q, kc, vc, bt, scale=SCALE, kv_scales=scales)
    torch.cuda.synchronize()
    ref_parts = [t.clone() for t in (static.part_m, static.part_l, static.part_o)]
    for i in range(launches):
        for t in (claimed.part_m, claimed.part_l, claimed.part_o):
            t.fill_(float("nan"))
        out = claimed(q, kc, vc, bt, scale=SCALE, kv_scales=scales)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"launch {i}: output differs from the static launch"
        for a, b in zip((claimed.part_m, claimed.part_l, claimed.part_o), ref_parts):
            assert torch.equal(a[:claimed.S], b[:claimed.S]), f"launch {i}: partials differ"
        assert claimed.claim_state.cpu().tolist() == [0, 0], "claim state not reset"
    got = ref_out.cpu().numpy()
    ref = (oracle_decode_fp8 if fp8 else oracle_decode)(wl, oracle_requests)
    for b, r in ref.items():
        assert_close(got[b], r, f"request {b} (L={wl.kv_lens[b]})")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("seed,batch,max_len,W,tile,resident", [
    (0, 6, 3000, 37, 512, 13), (1, 9, 5000, 200, 128, 64), (2, 5, 700, 7, 512, 1000), (3, 12, 9000, 64, 64, 256),
])
def test_claimed_equals_static(lb, fp8, seed, batch, max_len, W, tile, resident):
    wl = WL.random_decode(50 + seed, batch, max_len)
    wl.kv_lens[0] = 0                          # an empty request
    note(f"claimed fp8={fp8} lens={wl.kv_lens} W={W} tile={tile} resident={resident}")
    _compare(lb, wl, W, tile, resident, fp8)


@pytest.mark.parametrize("name,W,tile", [("long_tail", 512, 128), ("mixed_tp8", 2048, 128)])
def test_claimed_full_size(lb, name, W, tile):
    """The configurations the bench times: the long-tail batch and one GPU's 8-way KV-head share of
    the mixed batch, one resident wave per SIMD claiming finer lists; the long-tail batch's every
    request against the oracle, three requests of each length for the share."""
    wl = WL.BY_NAME[name]()
    resident = lb.attn_query_workers(0, 8) * 8
    note(f"claimed full size {name}: W={W} tile={tile} resident={resident}")
    if name == "long_tail":
        reqs = None
    else:
        reqs = [b for L in sorted(set(wl.kv_lens)) for b in [i for i, x in enumerate(wl.kv_lens) if x == L][:3]]
    _compare(lb, wl, W, tile, resident, False, launches=2, oracle_requests=reqs)
