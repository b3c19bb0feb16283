"""GPU parity against the fp64 oracle at KV-head counts other than 8 (query heads always 8 per KV
head): decode over the bf16 and E4M3 caches with every head-group split the kernel accepts (one
to eight KV heads per workgroup), and chunked prefill, whose grid pads the (worker, KV head) pairs
to whole XCD groups and whose combine takes the per-head form when there are not 64 query heads."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import (SCALE, assert_close, decode_inputs, decode_inputs_fp8, note, oracle_decode,
                         oracle_decode_fp8, prefill_inputs, q_starts)
from oracle.attention import ref_attention
from oracle.plan import ref_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("hkv,G", [(1, 1), (2, 1), (2, 2), (4, 1), (4, 4), (16, 2), (16, 4), (16, 16)])
def test_decode_head_counts(lb, hkv, G, fp8):
    from load_balanced_split_attn_amd import map_header
    wl = WL.random_decode(70 + hkv + G, 6, 2500, hq=8 * hkv, hkv=hkv)
    wl.kv_lens[0] = 0
    note(f"decode hkv={hkv} G={G} fp8={fp8} lens={wl.kv_lens}")
    W = 7
    words = lb.attn_plan(wl.kv_lens, W, 512)
    assert np.array_equal(words, ref_plan(wl.kv_lens, W, 512))
    if fp8:
        inputs = decode_inputs_fp8(wl, pad_code=0x7F)
        ref = oracle_decode_fp8(wl)
    else:
        inputs = decode_inputs(wl, pad_value=float("nan"))
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
        assert_close(got[b], ref[b], f"hkv {hkv} G {G} request {b} (L={wl.kv_lens[b]})")


def test_head_group_split_must_fit(lb):
    """A head-group count that does not divide the KV heads, or leaves a workgroup more than eight
    KV heads, is refused before any launch."""
    from load_balanced_split_attn_amd import LbsaError
    wl = WL.random_decode(90, 2, 300, hq=8 * 16, hkv=16)
    q, kc, vc, bt = decode_inputs(wl)
    words = lb.attn_plan(wl.kv_lens, 3, 512)
    mp = torch.from_numpy(np.asarray(words, dtype=np.int32)).to(q.device)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=q.device)
    S = max(int(words[4]), 1)
    pm = torch.empty((S, wl.hq), dtype=torch.float32, device=q.device)
    po = torch.empty((S, wl.hq, wl.head_dim), dtype=torch.float32, device=q.device)
    for G in (3, 1):   # 16 % 3 != 0; 16 KV heads in one workgroup
        with pytest.raises(LbsaError):
            lb.attn_splitkv(q, kc, vc, bt, lens, mp, 3, int(words[4]), G, SCALE, pm, pm.clone(), po)


@pytest.mark.parametrize("q_tile", [256, 128])
@pytest.mark.parametrize("hkv", [1, 2, 16])
def test_prefill_head_counts(hkv, q_tile):
    from load_balanced_split_attn_amd.prefill import PrefillStep
    wl = WL.random_prefill(80 + hkv, 3, 900, 300, hq=8 * hkv, hkv=hkv)
    note(f"prefill hkv={hkv} q_tile={q_tile} q_lens={wl.q_lens} kv_lens={wl.kv_lens}")
    q, kc, vc, bt = prefill_inputs(wl, pad_value=float("nan"))
    step = PrefillStep(wl.q_lens, wl.kv_lens, q.device, num_workers=5, num_q_heads=wl.hq, q_tile=q_tile)
    for t in (step.part_m, step.part_l, step.part_o):
        t.fill_(float("nan"))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    starts = q_starts(wl)
    for b in range(wl.batch):
        k, v = wl.kv(b)
        ref = ref_attention(wl.q(b).double().numpy(), k.double().numpy(), v.double().numpy(), SCALE, causal=True)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"prefill hkv {hkv} request {b}")
