"""GPU parity on inputs that make the online softmax move its reference maximum part-way through a
split, and on V values far from N(0, 1).

Splitting a request's keys over workers and merging the partials is an exact re-association of one
softmax sum ([P3] "Hy3 Preview AI Infra 推理优化精读笔记" §3.1 方案 step 5 and §14 "Split-KV").  The
kernels keep it exact with a lazy rescale: probabilities are taken against a reference maximum that
moves only when a chunk's largest score passes it by a slack, and then the accumulators are
rescaled.  N(0, 1) inputs never pass that slack after the first chunk, so these tests use the score
profiles of the workload generators (q scaled by 8 and 16, scores climbing along the sequence, late
dominant keys).  Each test first replays the kernels' rule on the host and asserts that rescales
from a finite reference happen in most segments and that, for some of them, the mass before the
rescale is a sizable share of the partial (so a wrong factor would show), then compares every
output element and every partial (m, lse, o/l) with the fp64 oracle."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import SCALE, assert_close, note, q_starts, rescale_replay
from oracle.attention import ref_attention, ref_split_partials
from oracle.fp8 import dequantize_kv
from oracle.plan import parse_map, ref_plan, ref_plan_prefill

pytestmark = pytest.mark.gpu

PEAKED = ["q8", "q16", "ramp", "spike"]
NAN_CODE = 0x7F


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _host_kv(wl, fp8):
    """Per request (k, v) as float64, dequantised for an 8-bit cache: what the kernels compute on."""
    if not fp8:
        return [tuple(t.double().numpy() for t in wl.kv(b)) for b in range(wl.batch)]
    ks, vs = (s.double().numpy() for s in wl.kv_scales())
    out = []
    for b in range(wl.batch):
        kc, vc = wl.kv_fp8(b)
        out.append((dequantize_kv(kc.numpy(), ks), dequantize_kv(vc.numpy(), vs)))
    return out


def _replay(words, q_rows, kvs, causal=True):
    """Host replay of the rescale rule over every segment of a map: (segments with a finite-reference
    rescale, segments with at least two chunks, largest pre-rescale share)."""
    mp = parse_map(words)
    hit = multi = 0
    frac = 0.0
    for b, i, a, e in mp.segs:
        b, i, a, e = int(b), int(i), int(a), int(e)
        qb = q_rows[b]
        r0, r1 = i * mp.q_tile, min(qb.shape[0], (i + 1) * mp.q_tile)
        if r1 <= r0 or e <= a:
            continue
        kv_len = kvs[b][0].shape[0]
        prefix = kv_len - qb.shape[0]
        vis = [prefix + j + 1 if causal else kv_len for j in range(r0, r1)]
        fin, _, f = rescale_replay(qb[r0:r1], kvs[b][0], a, e, vis, SCALE)
        if e - (a // 64) * 64 > 64:
            multi += 1
            hit += int(fin.sum() > 0)
        frac = max(frac, f)
    return hit, multi, frac


def _assert_rescales(words, q_rows, kvs, what, causal=True, min_share=1e-2):
    """Most multi-chunk segments rescale from a finite reference, and (min_share > 0) some rescale
    moves at least min_share of its partial's final sum.  The ramp profile climbs by more than the
    slack every chunk, so its earlier mass is tiny by construction: it is there for the count."""
    hit, multi, frac = _replay(words, q_rows, kvs, causal)
    note(f"  {what}: finite-reference rescales in {hit} of {multi} multi-chunk segments; "
         f"largest pre-rescale share {frac:.3g}")
    assert multi > 0 and 2 * hit > multi, f"{what}: rescales in only {hit} of {multi} segments"
    assert frac >= min_share, f"{what}: no rescale carries a sizable share of its partial ({frac:.2e})"


def _check_partials(words, q_rows, kvs, parts, rows_per_slot, causal=True):
    """Partial-level diagnostics per slot and stored row: m within 1e-3, lse within 1e-3, o / l at the
    output gates."""
    mp = parse_map(words)
    rparts = ref_split_partials(words, q_rows, [k for k, _ in kvs], [v for _, v in kvs], SCALE, causal)
    pm, pl, po = (t.cpu().numpy() for t in parts)
    pm = pm.reshape(pm.shape[0], rows_per_slot, -1)
    pl = pl.reshape(pl.shape[0], rows_per_slot, -1)
    po = po.reshape(po.shape[0], rows_per_slot, pm.shape[2], -1)
    for s, (m, l, o) in enumerate(rparts):
        n = m.shape[0]
        gm, gl, go = pm[s, :n], pl[s, :n], po[s, :n]
        fin = np.isfinite(m)
        assert np.array_equal(np.isfinite(gm), fin), f"slot {s}: empty rows differ"
        if not fin.any():
            continue
        assert np.max(np.abs(gm[fin] - m[fin])) <= 1e-3, f"slot {s} m"
        lse_g = gm[fin] + np.log(gl[fin])
        lse_r = m[fin] + np.log(l[fin])
        assert np.max(np.abs(lse_g - lse_r)) <= 1e-3, f"slot {s} lse"
        assert_close(go[fin] / gl[fin][:, None], o[fin] / l[fin][:, None], f"slot {s} o/l")
    assert len(rparts) == mp.S


def _decode_batch(profile):
    wl = WL.random_decode(21, 6, 6000, min_len=700)
    wl.profile = profile
    return wl


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("profile", PEAKED)
def test_decode_rescale(lb, profile, fp8):
    from gpu_helpers import decode_inputs, decode_inputs_fp8
    wl = _decode_batch(profile)
    W = 7
    note(f"decode rescale profile={profile} fp8={fp8} lens={wl.kv_lens} W={W}")
    words = lb.attn_plan(wl.kv_lens, W, 512)
    assert np.array_equal(words, ref_plan(wl.kv_lens, W, 512))
    q = wl.q().double().numpy()
    q_rows = [q[b:b + 1] for b in range(wl.batch)]
    kvs = _host_kv(wl, fp8)
    _assert_rescales(words, q_rows, kvs, f"decode {profile}", min_share=0 if profile == "ramp" else 1e-2)
    hdr = lb.map_header(words)
    dev = torch.device("cuda")
    S = hdr["S"]
    pm = torch.full((S, wl.hq), float("nan"), device=dev)
    pl = torch.full((S, wl.hq), float("nan"), device=dev)
    po = torch.full((S, wl.hq, wl.head_dim), float("nan"), device=dev)
    mp = torch.from_numpy(words).to(dev)
    lens = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    if fp8:
        qd, kc, vc, bt, ks, vs = decode_inputs_fp8(wl, pad_code=NAN_CODE)
        lb.attn_splitkv_fp8(qd, kc, vc, ks, vs, bt, lens, mp, W, S, 8, SCALE, pm, pl, po)
    else:
        qd, kc, vc, bt = decode_inputs(wl, pad_value=float("nan"))
        lb.attn_splitkv(qd, kc, vc, bt, lens, mp, W, S, 8, SCALE, pm, pl, po)
    out = torch.full(qd.shape, float("nan"), device=dev)
    lb.attn_combine(pm, pl, po, mp, hdr["U"], out, max_splits=lb.max_splits_of(words))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(wl.batch):
        ref = ref_attention(q_rows[b], kvs[b][0], kvs[b][1], SCALE)[0]
        assert_close(got[b], ref, f"{profile} request {b} (L={wl.kv_lens[b]})")
    _check_partials(words, q_rows, kvs, (pm, pl, po), 1)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("R", [2, 4])
@pytest.mark.parametrize("profile", PEAKED)
def test_mtp_rescale(lb, profile, R, fp8):
    from gpu_helpers import mtp_inputs
    from load_balanced_split_attn_amd.mtp import MtpDecodeStep
    wl = WL.random_mtp(31 + R, 5, 5000, max_q=R, min_len=700)
    wl.profile = profile
    wl.q_lens = [R, max(1, wl.q_lens[1]), R, wl.q_lens[3], R]
    W = 6
    note(f"mtp rescale profile={profile} R={R} fp8={fp8} kv={wl.kv_lens} q={wl.q_lens}")
    q_rows = [wl.q(b).double().numpy() for b in range(wl.batch)]
    kvs = _host_kv(wl, fp8)
    q, kc, vc, bt, scales = mtp_inputs(wl, fp8=fp8, pad=NAN_CODE if fp8 else float("nan"))
    step = MtpDecodeStep(wl.q_lens, wl.kv_lens, q.device, num_workers=W, tile=512,
                         kv_dtype=lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16)
    assert step.R == R
    assert np.array_equal(step.map_host, ref_plan_prefill(wl.q_lens, wl.kv_lens, W, R, 512, True))
    _assert_rescales(step.map_host, q_rows, kvs, f"mtp {profile} R={R}", min_share=0 if profile == "ramp" else 1e-2)
    for t in (step.part_m, step.part_l, step.part_o):
        t.fill_(float("nan"))
    out = torch.full(q.shape, float("nan"), device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out, kv_scales=scales)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    starts = q_starts(wl)
    for b in range(wl.batch):
        if wl.q_lens[b] == 0:
            continue
        ref = ref_attention(q_rows[b], kvs[b][0], kvs[b][1], SCALE, causal=True)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"{profile} R={R} request {b}")
    _check_partials(step.map_host, q_rows, kvs, (step.part_m, step.part_l, step.part_o), R)


def _run_prefill(lb, wl, W, q_tile, exact_pv, kvs, q_rows, replay=True):
    from gpu_helpers import prefill_inputs
    from load_balanced_split_attn_amd.prefill import PrefillStep
    q, kc, vc, bt = prefill_inputs(wl, pad_value=float("nan"))
    step = PrefillStep(wl.q_lens, wl.kv_lens, q.device, num_workers=W, q_tile=q_tile, exact_pv=exact_pv)
    assert np.array_equal(step.map_host, ref_plan_prefill(wl.q_lens, wl.kv_lens, W, q_tile, 512, True))
    if replay:
        _assert_rescales(step.map_host, q_rows, kvs, f"prefill {wl.profile} q_tile={q_tile}",
                         min_share=0 if wl.profile == "ramp" else 1e-2)
    for t in (step.part_m, step.part_l, step.part_o):
        t.fill_(float("nan"))
    out = torch.full(q.shape, float("nan"), device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), step


@pytest.mark.parametrize("q_tile", [128, 256])
@pytest.mark.parametrize("exact_pv", [None, True, False])
@pytest.mark.parametrize("profile", PEAKED)
def test_prefill_rescale(lb, profile, exact_pv, q_tile):
    wl = WL.random_prefill(41, 3, 2500, 300)
    wl.profile = profile
    W = 5
    note(f"prefill rescale profile={profile} exact_pv={exact_pv} q_tile={q_tile} q={wl.q_lens} kv={wl.kv_lens}")
    q_rows = [wl.q(b).double().numpy() for b in range(wl.batch)]
    kvs = _host_kv(wl, False)
    got, step = _run_prefill(lb, wl, W, q_tile, exact_pv, kvs, q_rows)
    starts = q_starts(wl)
    for b in range(wl.batch):
        ref = ref_attention(q_rows[b], kvs[b][0], kvs[b][1], SCALE, causal=True)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"{profile} request {b}")
    _check_partials(step.map_host, q_rows, kvs, (step.part_m, step.part_l, step.part_o), q_tile)


# ---- V far from N(0, 1) -----------------------------------------------------------------------

@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("profile", ["vsmall", "vlarge"])
def test_decode_value_range(lb, profile, fp8):
    """Decode carries bf16 V (or E4M3 codes times the V scale) exactly at any magnitude."""
    from load_balanced_split_attn_amd.decode import DecodeStep
    from gpu_helpers import decode_inputs, decode_inputs_fp8
    wl = _decode_batch(profile)
    note(f"decode value range {profile} fp8={fp8}")
    kvs = _host_kv(wl, fp8)
    q = wl.q().double().numpy()
    if fp8:
        qd, kc, vc, bt, ks, vs = decode_inputs_fp8(wl)
        step = DecodeStep(wl.kv_lens, qd.device, num_workers=7, kv_dtype=lb.KV_FP8_E4M3)
        out = step(qd, kc, vc, bt, scale=SCALE, kv_scales=(ks, vs))
    else:
        qd, kc, vc, bt = decode_inputs(wl)
        out = DecodeStep(wl.kv_lens, qd.device, num_workers=7)(qd, kc, vc, bt, scale=SCALE)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(wl.batch):
        ref = ref_attention(q[b:b + 1], kvs[b][0], kvs[b][1], SCALE)[0]
        assert_close(got[b], ref, f"{profile} request {b}", max_abs=1e-2 * float(np.max(np.abs(ref))))


@pytest.mark.parametrize("q_tile", [128, 256])
@pytest.mark.parametrize("profile", ["vsmall", "vlarge", "vlow", "vhigh"])
def test_prefill_exact_value_range(lb, profile, q_tile):
    """The default (exact) P.V path carries every bf16 V: 1e-6 and 1e5 included."""
    wl = WL.random_prefill(42, 3, 2500, 300)
    wl.profile = profile
    note(f"prefill exact P.V value range {profile} q_tile={q_tile}")
    q_rows = [wl.q(b).double().numpy() for b in range(wl.batch)]
    kvs = _host_kv(wl, False)
    got, _ = _run_prefill(lb, wl, 5, q_tile, True, kvs, q_rows, replay=False)
    starts = q_starts(wl)
    for b in range(wl.batch):
        ref = ref_attention(q_rows[b], kvs[b][0], kvs[b][1], SCALE, causal=True)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"{profile} request {b}",
                     max_abs=1e-2 * float(np.max(np.abs(ref))))


def _as_fp16_pv(v):
    """V as the fp16 P.V path holds it: rounded toward zero onto fp16 (spacing 2^-24 below 2^-14,
    bf16 values at or above 2^-17 unchanged), saturated at +-65504."""
    a = np.abs(v)
    sub = np.floor(a * 2.0 ** 24) / 2.0 ** 24
    return np.sign(v) * np.minimum(np.where(a < 2.0 ** -14, sub, a), 65504.0)


@pytest.mark.parametrize("q_tile", [128, 256])
@pytest.mark.parametrize("profile", ["vlow", "vhigh", "vsmall", "vlarge"])
def test_prefill_f16_value_range(lb, profile, q_tile):
    """The fp16 P.V path: with V of magnitude 2^-10 or 2^13 (nearly all inside the documented range
    2^-17 <= |v| <= 65504; vlow, vhigh) it matches the oracle on V itself; far outside it (vsmall,
    vlarge) it computes attention over V rounded toward zero onto fp16 and saturated, exactly as
    documented, and that is what the oracle is given."""
    wl = WL.random_prefill(42, 3, 2500, 300)
    wl.profile = profile
    note(f"prefill fp16 P.V value range {profile} q_tile={q_tile}")
    q_rows = [wl.q(b).double().numpy() for b in range(wl.batch)]
    kvs = _host_kv(wl, False)
    got, _ = _run_prefill(lb, wl, 5, q_tile, False, kvs, q_rows, replay=False)
    starts = q_starts(wl)
    for b in range(wl.batch):
        v = kvs[b][1] if profile in ("vlow", "vhigh") else _as_fp16_pv(kvs[b][1])
        ref = ref_attention(q_rows[b], kvs[b][0], v, SCALE, causal=True)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"{profile} request {b}",
                     max_abs=1e-2 * float(np.max(np.abs(ref))))


def _window_v(v: torch.Tensor, case: str, b: int) -> torch.Tensor:
    """V for the window test: magnitudes drawn from the case's range, signs from v (bf16)."""
    g = torch.Generator().manual_seed(1234 + b)
    u = torch.rand(v.shape, generator=g, dtype=torch.float32)
    sign = torch.where(v.float() < 0, -1.0, 1.0)
    if case == "lo_in":        # [2^-23, 2^-22): the smallest magnitudes the fp16 copy holds
        mag = 2.0 ** -23 * (1.0 + u)
    elif case == "lo_out":     # [2^-24, 2^-23): every chunk stamped
        mag = 2.0 ** -24 * (1.0 + u)
    elif case == "hi_in":      # [510, 1015]: up to the largest magnitudes the fp16 copy holds
        mag = 510.0 * (1.0 + 0.99 * u)
    elif case == "hi_out":     # [1024, 2048): every chunk stamped
        mag = 1024.0 * (1.0 + u)
    else:                      # "sigma": N(0, 0.02^2), the shift's reason
        return (v.float() * 0.02).to(torch.bfloat16)
    return (sign * mag).to(torch.bfloat16)


@pytest.mark.parametrize("q_tile", [128, 256])
@pytest.mark.parametrize("case", ["lo_in", "lo_out", "hi_in", "hi_out", "sigma"])
def test_prefill_checked_window_edges(lb, case, q_tile):
    """The default P.V carries V * 2^6 in fp16 for 2^-23 <= |v| <= 1020 and stamps any chunk with a
    value outside: V just inside and just outside each end of that window, and N(0, 0.02^2) V,
    against the oracle on V itself."""
    wl = WL.random_prefill(43, 3, 2500, 300)
    base = wl.kv

    def kv(b, base=base):
        k, v = base(b)
        return k, _window_v(v, case, b)

    wl.kv = kv
    note(f"prefill checked P.V window {case} q_tile={q_tile}")
    q_rows = [wl.q(b).double().numpy() for b in range(wl.batch)]
    kvs = _host_kv(wl, False)
    got, _ = _run_prefill(lb, wl, 5, q_tile, None, kvs, q_rows, replay=False)
    starts = q_starts(wl)
    for b in range(wl.batch):
        ref = ref_attention(q_rows[b], kvs[b][0], kvs[b][1], SCALE, causal=True)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"{case} request {b}",
                     max_abs=1e-2 * float(np.max(np.abs(ref))))


@pytest.mark.parametrize("q_tile", [128, 256])
@pytest.mark.parametrize("profile", ["vsmall", "vlarge", "vlow", "vhigh", "outlier"])
def test_prefill_checked_value_range(lb, profile, q_tile):
    """The default P.V path (fp16 on checked chunks, bf16 for a chunk fp16 does not hold exactly)
    carries V exactly for every input: V scaled by 1e-6, 1e5, 2^-10, 2^13, and N(0, 1) values with a
    single 1e5 among them, each against the oracle on V itself (not on V as fp16 would hold it)."""
    wl = WL.random_prefill(42, 3, 2500, 300)
    if profile == "outlier":
        base = wl.kv

        def kv(b, base=base):
            k, v = base(b)
            if b == 1:
                v = v.clone()
                v[700, 3, 17] = 1e5
            return k, v

        wl.kv = kv
    else:
        wl.profile = profile
    note(f"prefill checked P.V value range {profile} q_tile={q_tile}")
    q_rows = [wl.q(b).double().numpy() for b in range(wl.batch)]
    kvs = _host_kv(wl, False)
    got, _ = _run_prefill(lb, wl, 5, q_tile, None, kvs, q_rows, replay=False)
    starts = q_starts(wl)
    for b in range(wl.batch):
        ref = ref_attention(q_rows[b], kvs[b][0], kvs[b][1], SCALE, causal=True)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"{profile} request {b}",
                     max_abs=1e-2 * float(np.max(np.abs(ref))))
