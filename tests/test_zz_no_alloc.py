"""The allocation-free decode entry point (attn_decode_noalloc, partials in the library's fixed
device array) against the allocating path it mirrors (attn_splitkv / attn_splitkv_fp8 +
attn_combine with caller-owned partials) and the fp64 oracle, on two calls in a row, the second
with a smaller batch; a call whose partials would not fit is refused before any launch."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import SCALE, assert_close, decode_inputs, decode_inputs_fp8, note, oracle_decode, oracle_decode_fp8
from oracle.plan import ref_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _both(lb, wl, W, fp8, out_dtype):
    """(noalloc output, allocating-path output) for one batch."""
    words = lb.attn_plan(wl.kv_lens, W, 512)
    assert np.array_equal(words, ref_plan(wl.kv_lens, W, 512))
    hdr = lb.map_header(words)
    if fp8:
        q, kc, vc, bt, ks, vs = decode_inputs_fp8(wl)
    else:
        q, kc, vc, bt = decode_inputs(wl)
        ks = vs = None
    dev = q.device
    mp = torch.from_numpy(words).to(dev)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    S, ms = hdr["S"], lb.max_splits_of(words)
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=dev)
    lb.attn_decode_noalloc(q, kc, vc, bt, lens, mp, W, S, 8, SCALE, out, max_splits=ms,
                           kv_scales=(ks, vs) if fp8 else None)
    pm = torch.empty((S, wl.hq), device=dev)
    pl = torch.empty((S, wl.hq), device=dev)
    po = torch.empty((S, wl.hq, wl.head_dim), device=dev)
    if fp8:
        lb.attn_splitkv_fp8(q, kc, vc, ks, vs, bt, lens, mp, W, S, 8, SCALE, pm, pl, po)
    else:
        lb.attn_splitkv(q, kc, vc, bt, lens, mp, W, S, 8, SCALE, pm, pl, po)
    ref_out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=dev)
    lb.attn_combine(pm, pl, po, mp, hdr["U"], ref_out, max_splits=ms)
    torch.cuda.synchronize()
    return out, ref_out


@pytest.mark.parametrize("fp8", [False, True])
def test_noalloc_two_calls_second_smaller(lb, fp8):
    first = WL.random_decode(61, 9, 9000, min_len=1)
    second = WL.random_decode(62, 4, 3000, min_len=1)
    for wl, W, out_dtype in ((first, 40, torch.float32), (second, 11, torch.bfloat16)):
        note(f"noalloc fp8={fp8} lens={wl.kv_lens} W={W} out={out_dtype}")
        out, ref_out = _both(lb, wl, W, fp8, out_dtype)
        assert torch.equal(out, ref_out), "noalloc output differs from the allocating path"
        ref = oracle_decode_fp8(wl) if fp8 else oracle_decode(wl)
        got = out.float().cpu().numpy()
        for b in range(wl.batch):
            assert_close(got[b], ref[b], f"request {b}")


def test_noalloc_graph_replays(lb):
    """The allocation-free step captured in a HIP graph (its first call, which resolves the array's
    device address, made before the capture): three replays with new query values, each bit for
    bit equal to the allocating path on the same inputs."""
    wl = WL.random_decode(64, 6, 5000, min_len=1)
    W = 24
    words = lb.attn_plan(wl.kv_lens, W, 512)
    hdr = lb.map_header(words)
    q, kc, vc, bt = decode_inputs(wl)
    dev = q.device
    mp = torch.from_numpy(words).to(dev)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    S, ms = hdr["S"], lb.max_splits_of(words)
    out = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    pm = torch.empty((S, wl.hq), device=dev)
    pl = torch.empty((S, wl.hq), device=dev)
    po = torch.empty((S, wl.hq, wl.head_dim), device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lb.attn_decode_noalloc(q, kc, vc, bt, lens, mp, W, S, 8, SCALE, out, max_splits=ms)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lb.attn_decode_noalloc(q, kc, vc, bt, lens, mp, W, S, 8, SCALE, out, max_splits=ms)
    torch.cuda.synchronize()
    q0 = q.clone()
    for replay in range(3):
        q.copy_((q0.float() * (1.0 + 0.5 * replay)).to(torch.bfloat16))
        ref_out = torch.full(q.shape, float("nan"), device=dev)
        lb.attn_splitkv(q, kc, vc, bt, lens, mp, W, S, 8, SCALE, pm, pl, po)
        lb.attn_combine(pm, pl, po, mp, hdr["U"], ref_out, max_splits=ms)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {replay}: noalloc graph output differs"
        note(f"noalloc graph replay {replay} ok")


def test_noalloc_refuses_oversized_partials(lb):
    """More segments than the array holds: LBSA_ERR_CAPACITY, nothing launched."""
    wl = WL.random_decode(63, 2, 600, min_len=1)
    q, kc, vc, bt = decode_inputs(wl)
    words = lb.attn_plan(wl.kv_lens, 2, 512)
    mp = torch.from_numpy(words).to(q.device)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=q.device)
    out = torch.zeros(q.shape, device=q.device)
    too_many = lb.NOALLOC_SCRATCH_BYTES // (wl.hq * (wl.head_dim + 2) * 4) + 1
    with pytest.raises(lb.LbsaError) as e:
        lb.attn_decode_noalloc(q, kc, vc, bt, lens, mp, 2, too_many, 8, SCALE, out)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
