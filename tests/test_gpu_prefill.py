"""GPU parity of the chunked-prefill path (attn_plan_prefill -> attn_splitkv_prefill ->
attn_combine through the C ABI) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import (SCALE, assert_close, errors, note, oracle_prefill_rows, prefill_inputs, q_starts)
from oracle.attention import ref_attention
from oracle.plan import ref_plan_prefill

pytestmark = pytest.mark.gpu


def _run(wl, W, causal=True, inputs=None, poison=False, kv_tile=512, exact_pv=None, q_tile=256):
    from load_balanced_split_attn_amd.prefill import PrefillStep
    q, kc, vc, bt = inputs if inputs is not None else prefill_inputs(wl, pad_value=float("nan"))
    step = PrefillStep(wl.q_lens, wl.kv_lens, q.device, num_workers=W, causal=causal, kv_tile=kv_tile,
                       exact_pv=exact_pv, q_tile=q_tile)
    assert np.array_equal(step.map_host, ref_plan_prefill(wl.q_lens, wl.kv_lens, W, q_tile, kv_tile, causal))
    if poison:
        for t in (step.part_m, step.part_l, step.part_o):
            t.fill_(float("nan"))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), step


def _check_all(wl, got, causal=True):
    starts = q_starts(wl)
    for b in range(wl.batch):
        k, v = wl.kv(b)
        ref = ref_attention(wl.q(b).double().numpy(), k.double().numpy(), v.double().numpy(), SCALE, causal=causal)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref,
                     f"{wl.name} request {b} (q_len={wl.q_lens[b]}, kv_len={wl.kv_lens[b]}, causal={causal})")


@pytest.mark.parametrize("q_tile", [256, 128])
@pytest.mark.parametrize("exact_pv", [None, False, True])
@pytest.mark.parametrize("seed,batch,max_prefix,max_chunk,W", [
    (0, 3, 1500, 300, 3), (1, 4, 700, 200, 1), (2, 2, 3000, 260, 8), (3, 5, 100, 140, 16),
])
def test_random_prefill(seed, batch, max_prefix, max_chunk, W, exact_pv, q_tile):
    wl = WL.random_prefill(seed, batch, max_prefix, max_chunk)
    note(f"prefill seed={seed} q_lens={wl.q_lens} kv_lens={wl.kv_lens} W={W} exact_pv={exact_pv} q_tile={q_tile}")
    got, _ = _run(wl, W, causal=True, poison=True, exact_pv=exact_pv, q_tile=q_tile)
    _check_all(wl, got, causal=True)


def test_non_causal_and_small_tiles():
    wl = WL.random_prefill(7, 3, 900, 200)
    note(f"non-causal q_lens={wl.q_lens} kv_lens={wl.kv_lens}")
    got, _ = _run(wl, 5, causal=False, exact_pv=False)
    _check_all(wl, got, causal=False)
    got, _ = _run(wl, 5, causal=False, exact_pv=True)
    _check_all(wl, got, causal=False)
    got, _ = _run(wl, 5, causal=True, kv_tile=64)
    _check_all(wl, got, causal=True)


def test_no_prefix_is_textbook_causal():
    wl = WL.random_prefill(8, 2, 0, 300)   # prefix 0: plain causal self-attention of the chunk
    note(f"no prefix q_lens={wl.q_lens} kv_lens={wl.kv_lens}")
    got, _ = _run(wl, 4)
    _check_all(wl, got)


@pytest.mark.parametrize("exact_pv", [None, False, True])
def test_segment_boundary_inside_a_wave(exact_pv):
    """Regression: a 128-row chunk after a 1000-token prefix sees keys up to 1000..1127, so the
    worker boundary at key 1024 (three 512-key tiles, one per worker) falls inside the rows of the
    first wave.  In the last segment rows 0..23 of that wave see no key while rows 24..31 do; the
    rows without a key must keep an empty partial while the others rescale."""
    wl = WL.Workload("boundary_in_wave", 250, [1128, 700], [128, 60], kind="prefill",
                     meta={"prefix": [1000, 640]})
    note(f"segment boundary inside a wave, exact_pv={exact_pv}")
    got, step = _run(wl, 3, poison=True, exact_pv=exact_pv)
    segs = step.map_host[-4 * step.S:].reshape(-1, 4)
    assert any(s[0] == 0 and s[2] == 1024 for s in segs)
    _check_all(wl, got)


def test_exact_pv_agrees_with_fp16_pv():
    """Both P.V precisions give the same attention to well inside the tolerance."""
    wl = WL.random_prefill(10, 3, 2500, 300)
    inputs = prefill_inputs(wl)
    a, _ = _run(wl, 6, inputs=inputs, exact_pv=False)
    b, _ = _run(wl, 6, inputs=inputs, exact_pv=True)
    assert errors(a.astype(np.float64), b.astype(np.float64))[1] <= 1e-3


def test_flags_rejected():
    import load_balanced_split_attn_amd as lb
    wl = WL.random_prefill(11, 1, 100, 50)
    q, kc, vc, bt = prefill_inputs(wl)
    from load_balanced_split_attn_amd.prefill import PrefillStep
    st = PrefillStep(wl.q_lens, wl.kv_lens, q.device, num_workers=2)
    lib = lb.lib()
    rc = lib.attn_splitkv_prefill(lb._dptr(q), lb._dptr(kc), lb._dptr(vc), lb._dptr(bt), bt.shape[1], kc.shape[0],
                                  lb._dptr(st.q_lens), lb._dptr(st.q_start), lb._dptr(st.kv_lens), lb._dptr(st.map),
                                  st.W, st.S, 1, 64, 8, 128, 64, 128, 1, SCALE, lb._dptr(st.part_m),
                                  lb._dptr(st.part_l), lb._dptr(st.part_o), 4, None)
    assert rc == -1
    rc = lib.attn_splitkv_prefill(lb._dptr(q), lb._dptr(kc), lb._dptr(vc), lb._dptr(bt), bt.shape[1], kc.shape[0],
                                  lb._dptr(st.q_lens), lb._dptr(st.q_start), lb._dptr(st.kv_lens), lb._dptr(st.map),
                                  st.W, st.S, 1, 64, 8, 128, 64, 128, 1, SCALE, lb._dptr(st.part_m),
                                  lb._dptr(st.part_l), lb._dptr(st.part_o), 3, None)
    assert rc == -1     # both precision flags at once


def test_single_row_matches_decode():
    """A one-row chunk is a decode query at the last position."""
    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.decode import DecodeStep
    wl = WL.random_prefill(9, 3, 2000, 1)
    wl.q_lens = [1] * wl.batch
    wl.kv_lens = [max(1, L) for L in wl.kv_lens]
    q, kc, vc, bt = prefill_inputs(wl)
    step = DecodeStep(wl.kv_lens, q.device, num_workers=3)
    dec = step(q, kc, vc, bt, scale=SCALE)
    torch.cuda.synchronize()
    dec = dec.cpu().numpy().astype(np.float64)
    exact, _ = _run(wl, 3, inputs=(q, kc, vc, bt), exact_pv=True)
    assert errors(exact.astype(np.float64), dec)[1] <= 1e-5          # same arithmetic up to fp32 order
    fast, _ = _run(wl, 3, inputs=(q, kc, vc, bt), exact_pv=False)
    assert errors(fast.astype(np.float64), dec)[1] <= 1e-3           # P rounded to fp16


@pytest.fixture(scope="module")
def full_prefill():
    """The chunked-prefill batch's inputs on the device and the fp64 oracle for (a) sampled rows of
    every request and (b) every row of the two requests with the shortest prefixes."""
    wl = WL.prefill()
    # every 37th row (all offsets inside a wave's 32 rows and a unit's 256 come up) plus both sides
    # of each 128-row unit boundary and the last row
    rows = sorted(set(range(0, 2048, 37)) | {u * 128 + d for u in range(1, 16) for d in (-1, 0)} | {2047})
    prefix = wl.meta["prefix"]
    whole = sorted(range(wl.batch), key=lambda b: prefix[b])[:2]
    sampled, full = {}, {}
    for b in range(wl.batch):
        if b in whole:
            k, v = wl.kv(b)
            full[b] = ref_attention(wl.q(b).double().numpy(), k.double().numpy(), v.double().numpy(), SCALE)
        else:
            sampled[b] = oracle_prefill_rows(wl, b, rows)
    note(f"full-size prefill oracle ready: every row of requests {whole} (prefixes "
         f"{[prefix[b] for b in whole]}), {len(rows)} sampled rows of the others")
    return wl, prefill_inputs(wl, pad_value=float("nan")), rows, sampled, full


@pytest.mark.parametrize("q_tile,exact_pv", [(128, None), (256, None), (128, True), (256, True), (128, False),
                                             (256, False)])
def test_full_size_prefill(full_prefill, q_tile, exact_pv):
    """The chunked-prefill batch (8 x 2048-row chunks after log-uniform [8K, 128K] prefixes) in each
    launch configuration the bench times (64 workers; 128- or 256-row units; checked-fp16, exact or fp16 P.V):
    every row of the two shortest-prefix requests and sampled rows of the others against the fp64
    oracle."""
    wl, inputs, rows, sampled, full = full_prefill
    note(f"full-size prefill q_tile={q_tile} exact_pv={exact_pv}")
    got, step = _run(wl, 64, inputs=inputs, poison=True, exact_pv=exact_pv, q_tile=q_tile)
    assert np.all(np.isfinite(got))
    starts = q_starts(wl)
    for b in range(wl.batch):
        if b in full:
            ma, rr = assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], full[b], f"prefill request {b}, all rows")
            worst = max(errors(got[starts[b] + j], full[b][j])[1] for j in range(wl.q_lens[b]))
            note(f"  request {b} kv_len={wl.kv_lens[b]}: all {wl.q_lens[b]} rows, rel_rms {rr:.2e} "
                 f"(worst row {worst:.2e})")
            for j in range(wl.q_lens[b]):
                assert_close(got[starts[b] + j], full[b][j], f"prefill request {b} row {j}")
        else:
            worst = 0.0
            for j in rows:
                ma, rr = assert_close(got[starts[b] + j], sampled[b][j], f"prefill request {b} row {j}")
                worst = max(worst, rr)
            note(f"  request {b} kv_len={wl.kv_lens[b]}: {len(rows)} rows ok (worst rel_rms {worst:.2e})")


def test_million_token_prefix_sampled():
    """Maximum-size prefill: a 2048-row causal chunk after a prefix of 2^20 - 2048 tokens (16,384
    pages, cache offsets past 2^31 bytes) beside a short request, in the bench launch (256-row
    units, 64 workers); sampled rows of the long request and every row of the short one against the
    fp64 oracle."""
    wl = WL.random_prefill(30, 2, 1000, 300)
    wl.q_lens[0] = 2048
    wl.kv_lens[0] = 1 << 20
    note(f"million-token prefill: q_lens={wl.q_lens} kv_lens={wl.kv_lens}")
    got, step = _run(wl, 64, poison=True)
    assert np.all(np.isfinite(got))
    starts = q_starts(wl)
    rows = [0, 1, 255, 256, 1023, 2047]
    ref = oracle_prefill_rows(wl, 0, rows)
    for j in rows:
        ma, rr = assert_close(got[starts[0] + j], ref[j], f"long request row {j}")
    note(f"  long request rows {rows} ok (last rel_rms {rr:.2e})")
    short = list(range(wl.q_lens[1]))
    ref = oracle_prefill_rows(wl, 1, short)
    for j in short:
        assert_close(got[starts[1] + j], ref[j], f"short request row {j}")


def test_unit_height_mismatch_writes_nothing():
    """A map planned for 128-row units given to the 256-row kernel is skipped, not misread."""
    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.prefill import PrefillStep
    wl = WL.random_prefill(12, 2, 300, 200)
    q, kc, vc, bt = prefill_inputs(wl)
    st = PrefillStep(wl.q_lens, wl.kv_lens, q.device, num_workers=2, q_tile=128)   # 128-row map
    S = max(st.S, 1)
    pm = torch.full((S, 256, 64), 7.0, device=q.device)
    pl = torch.full((S, 256, 64), 7.0, device=q.device)
    po = torch.full((S, 256, 64, 128), 7.0, device=q.device)
    lb.attn_splitkv_prefill(q, kc, vc, bt, st.q_lens, st.q_start, st.kv_lens, st.map, st.W, st.S, SCALE,
                            pm, pl, po, q_tile=256)
    torch.cuda.synchronize()
    assert bool((pm == 7.0).all()) and bool((pl == 7.0).all()) and bool((po == 7.0).all())


@pytest.mark.parametrize("q_tile", [256, 128])
def test_bf16_output_is_rounded_fp32_output(q_tile):
    """The combine run twice on the same partials: its bf16 output is its fp32 output rounded to
    nearest even, bit for bit, on every row of a ragged batch (the combine's store path for bf16)."""
    from load_balanced_split_attn_amd.prefill import PrefillStep
    wl = WL.random_prefill(7, 4, 1200, 300)
    note(f"bf16 out q_tile={q_tile} q_lens={wl.q_lens} kv_lens={wl.kv_lens}")
    q, kc, vc, bt = prefill_inputs(wl, pad_value=float("nan"))
    step = PrefillStep(wl.q_lens, wl.kv_lens, q.device, num_workers=5, q_tile=q_tile)
    step.splitkv(q, kc, vc, bt, SCALE)
    o32 = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    o16 = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    step.combine(o32)
    step.combine(o16)
    torch.cuda.synchronize()
    assert not torch.isnan(o32).any()
    assert torch.equal(o16.view(torch.int16).cpu(), o32.to(torch.bfloat16).view(torch.int16).cpu())
    _check_all(wl, o32.cpu().numpy())


@pytest.mark.parametrize("launch_workers", [3, 1])
def test_worker_count_mismatch_writes_nothing(launch_workers):
    """A map planned for two workers launched with another worker count is skipped on the device
    (its lists are never read past their end), for a larger and a smaller grid."""
    import load_balanced_split_attn_amd as lb
    from load_balanced_split_attn_amd.prefill import PrefillStep
    wl = WL.random_prefill(13, 2, 300, 200)
    q, kc, vc, bt = prefill_inputs(wl)
    st = PrefillStep(wl.q_lens, wl.kv_lens, q.device, num_workers=2)
    S = max(st.S, 1)
    pm = torch.full((S, 256, 64), 7.0, device=q.device)
    pl = torch.full((S, 256, 64), 7.0, device=q.device)
    po = torch.full((S, 256, 64, 128), 7.0, device=q.device)
    lb.attn_splitkv_prefill(q, kc, vc, bt, st.q_lens, st.q_start, st.kv_lens, st.map, launch_workers, st.S, SCALE,
                            pm, pl, po)
    torch.cuda.synchronize()
    assert bool((pm == 7.0).all()) and bool((pl == 7.0).all()) and bool((po == 7.0).all())


@pytest.mark.parametrize("q_tile", [128, 256])
def test_graph_captured_prefill_step(q_tile):
    """The prefill step (split-KV and combine on one stream) captured in a HIP graph: four replays
    with new query and key values written in place between them, and eager work of the program in
    between, each replay bit for bit equal to the eager step on the same inputs and within the gates
    of the fp64 oracle."""
    from load_balanced_split_attn_amd.prefill import PrefillStep
    wl = WL.random_prefill(77, 3, 2000, 300)
    q, kc, vc, bt = prefill_inputs(wl, pad_value=float("nan"))
    dev = q.device
    step = PrefillStep(wl.q_lens, wl.kv_lens, dev, num_workers=6, q_tile=q_tile)
    out = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                           # warm-up outside the capture
        step(q, kc, vc, bt, scale=SCALE, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q, kc, vc, bt, scale=SCALE, out=out)
    torch.cuda.synchronize()
    q0 = q.clone()
    gen = torch.Generator(device="cpu").manual_seed(11)
    starts = q_starts(wl)
    for replay in range(4):
        # new query rows (the scaled first rows; replay 0 keeps them) and the eager step beside the graph
        factor = 1.0 + 0.25 * replay
        q.copy_((q0.float() * factor).to(torch.bfloat16))
        eager = torch.empty_like(out)
        step(q, kc, vc, bt, scale=SCALE, out=eager)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        junk = torch.randn(1 << 16, generator=gen).to(dev).sum()      # the program's own eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, eager), f"replay {replay}: graph output differs from the eager step"
        got = out.cpu().numpy()
        qh = q.cpu()
        for b in range(wl.batch):
            k, v = wl.kv(b)
            rows = qh[starts[b]:starts[b] + wl.q_lens[b]].double().numpy()
            ref = ref_attention(rows, k.double().numpy(), v.double().numpy(), SCALE, causal=True)
            assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"replay {replay} request {b}")
        note(f"prefill graph replay {replay} (q x {factor}) ok")
