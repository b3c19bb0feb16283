"""GPU parity of multi-token decode (attn_plan_prefill with q_tile = R -> attn_splitkv_mtp ->
attn_combine through the C ABI) against the fp64 oracle: each request's q_len rows are the last
q_len positions of its context, causal among themselves; bf16 and 8-bit caches."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import SCALE, assert_close, errors, mtp_inputs, note, oracle_mtp, q_starts
from oracle.plan import ref_plan_prefill

pytestmark = pytest.mark.gpu

NAN_BF16 = float("nan")
NAN_CODE = 0x7F


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _run(lb, wl, W, G, fp8, inputs=None, poison=True, tile=512):
    from load_balanced_split_attn_amd.mtp import MtpDecodeStep
    q, kc, vc, bt, scales = inputs if inputs is not None else mtp_inputs(
        wl, fp8=fp8, pad=(NAN_CODE if fp8 else NAN_BF16) if poison else 0)
    step = MtpDecodeStep(wl.q_lens, wl.kv_lens, q.device, num_workers=W, tile=tile, head_groups=G,
                         kv_dtype=lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16)
    assert np.array_equal(step.map_host, ref_plan_prefill(wl.q_lens, wl.kv_lens, W, step.R, tile, True))
    if poison:
        for t in (step.part_m, step.part_l, step.part_o):
            t.fill_(float("nan"))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out, kv_scales=scales)
    torch.cuda.synchronize()
    return out.cpu().numpy(), step


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("seed,batch,max_len,W,G", [
    (0, 6, 3000, 7, 8), (1, 9, 1500, 1, 8), (2, 5, 5000, 64, 4), (3, 12, 700, 100, 2), (4, 4, 2600, 3, 1),
])
def test_random_ragged_mtp(lb, fp8, seed, batch, max_len, W, G):
    wl = WL.random_mtp(seed, batch, max_len)
    wl.q_lens[-1] = 4                               # at least one request with the full 4 rows
    wl.kv_lens[0] = max(wl.kv_lens[0], 513)         # a ragged tail past one tile
    note(f"mtp fp8={fp8} seed={seed} kv={wl.kv_lens} q={wl.q_lens} W={W} G={G}")
    got, _ = _run(lb, wl, W, G, fp8)
    ref = oracle_mtp(wl, fp8=fp8)
    starts = q_starts(wl)
    for b, r in ref.items():
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], r, f"request {b} (L={wl.kv_lens[b]}, q={wl.q_lens[b]})")


@pytest.mark.parametrize("q_len", [1, 2, 3])
def test_uniform_rows(lb, q_len):
    """All requests with the same row count (R = 1, 2, 3: one and two column blocks), short contexts
    so the causal edge falls inside the first chunk too."""
    wl = WL.random_mtp(7 + q_len, 8, 900, min_len=q_len)
    wl.q_lens = [q_len] * wl.batch
    wl.kv_lens[1] = q_len                           # the whole context is the drafted tokens
    got, step = _run(lb, wl, 13, 8, False)
    assert step.R == q_len
    ref = oracle_mtp(wl)
    starts = q_starts(wl)
    for b, r in ref.items():
        assert_close(got[starts[b]:starts[b] + q_len], r, f"q_len {q_len} request {b}")


def test_single_row_equals_plain_decode(lb):
    """q_len = 1 everywhere: the multi-token path equals the plain decode path."""
    from load_balanced_split_attn_amd.decode import DecodeStep
    wl = WL.random_mtp(20, 7, 4000, min_len=1)
    wl.q_lens = [1] * wl.batch
    inputs = mtp_inputs(wl)
    got, _ = _run(lb, wl, 37, 8, False, inputs=inputs, poison=False)
    q, kc, vc, bt, _ = inputs
    dec = DecodeStep(wl.kv_lens, q.device, num_workers=37, head_groups=8)(q, kc, vc, bt, scale=SCALE)
    torch.cuda.synchronize()
    assert errors(got.astype(np.float64), dec.cpu().numpy().astype(np.float64))[1] <= 1e-6


@pytest.mark.parametrize("fp8", [False, True])
def test_full_size_mtp4_mixed(lb, fp8):
    """The mixed batch with 4 drafted tokens per request in the bench launch configuration; every
    request against the oracle."""
    wl = WL.mtp(4)
    note(f"full-size mtp4 mixed fp8={fp8}")
    W = lb.attn_query_workers(0, 8, lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16)
    got, _ = _run(lb, wl, W, 8, fp8, poison=False)
    assert np.all(np.isfinite(got))
    starts = q_starts(wl)
    worst = (0.0, 0.0)
    for b in range(wl.batch):
        r = oracle_mtp(wl, [b], fp8=fp8)[b]
        ma, rr = assert_close(got[starts[b]:starts[b] + 4], r, f"mtp4 request {b} (L={wl.kv_lens[b]})")
        worst = (max(worst[0], ma), max(worst[1], rr))
    note(f"  all {wl.batch} requests: worst max_abs={worst[0]:.2e} rel_rms={worst[1]:.2e}")


@pytest.mark.parametrize("fp8", [False, True])
def test_graph_captured_mtp_step(lb, fp8):
    """The multi-token decode step (split-KV and combine) captured in a HIP graph: four replays with
    new query rows written in place and the program's own eager work between them, each bit for bit
    equal to the eager step on the same inputs; the first replay also against the fp64 oracle."""
    from load_balanced_split_attn_amd.mtp import MtpDecodeStep
    wl = WL.random_mtp(41, 7, 2600)
    wl.q_lens[-1] = 4
    q, kc, vc, bt, scales = mtp_inputs(wl, fp8=fp8, pad=NAN_CODE if fp8 else NAN_BF16)
    step = MtpDecodeStep(wl.q_lens, wl.kv_lens, q.device, num_workers=9,
                         kv_dtype=lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16)
    out = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                           # warm-up outside the capture
        step(q, kc, vc, bt, scale=SCALE, out=out, kv_scales=scales)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q, kc, vc, bt, scale=SCALE, out=out, kv_scales=scales)
    torch.cuda.synchronize()
    q0 = q.clone()
    starts = q_starts(wl)
    for replay in range(4):
        q.copy_((q0.float() * (1.0 + 0.5 * replay)).to(torch.bfloat16))
        eager = torch.empty_like(out)
        step(q, kc, vc, bt, scale=SCALE, out=eager, kv_scales=scales)
        junk = torch.randn(1 << 16, device=q.device).sum()   # the program's own eager work
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, eager), f"replay {replay}: graph output differs from the eager step"
        if replay == 0:
            got = out.cpu().numpy()
            for b, r in oracle_mtp(wl, fp8=fp8).items():
                assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], r, f"request {b}")
        note(f"mtp graph replay {replay} ok")


@pytest.mark.parametrize("R,G", [(2, 8), (4, 8), (3, 4)])
def test_launch_order_bitwise(lb, R, G):
    """The multi-token step's map launched head-major and list-major: the same output bit for bit
    (the host map is the oracle's either way)."""
    from load_balanced_split_attn_amd.mtp import MtpDecodeStep
    wl = WL.random_mtp(300 + R, 13, 6000, max_q=R)
    inputs = mtp_inputs(wl)
    q, kc, vc, bt, scales = inputs
    note(f"mtp launch order R={R} G={G}")
    outs = []
    for order in ("head", "list"):
        step = MtpDecodeStep(wl.q_lens, wl.kv_lens, q.device, num_workers=16, head_groups=G, launch_order=order)
        assert np.array_equal(step.map_host, ref_plan_prefill(wl.q_lens, wl.kv_lens, 16, step.R, 512, True))
        assert step.list_major == (order == "list")
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
        outs.append(step(q, kc, vc, bt, scale=SCALE, out=out))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    ref = oracle_mtp(wl)
    starts = q_starts(wl)
    for b, rows in ref.items():
        assert_close(outs[1][starts[b]:starts[b] + wl.q_lens[b]].cpu().numpy(), rows, f"mtp request {b}")
