"""GPU parity against the fp64 oracle, with NaN-poisoned pads, at cache page sizes other than 64
tokens (any multiple of 64 is accepted) and on a batch of many small requests.  With pages of 128,
256 and 1024 tokens the decode kernels (bf16 and E4M3), multi-token decode, chunked prefill and the
producer step walk several 64-token chunks per page and start segments inside a page."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import (SCALE, assert_close, decode_inputs, decode_inputs_fp8, mtp_inputs, note, oracle_decode,
                         oracle_decode_fp8, oracle_mtp, prefill_inputs, q_starts)
from oracle.attention import ref_attention
from oracle.plan import ref_plan, ref_plan_prefill

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _decode(lb, wl, words, inputs, G, fp8):
    from load_balanced_split_attn_amd import map_header
    q, kc, vc, bt = inputs[:4]
    hdr = map_header(words)
    dev = q.device
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
    return out.cpu().numpy()


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("page,G,tile", [(128, 8, 512), (256, 4, 512), (1024, 8, 512), (256, 8, 64)])
def test_decode_page_sizes(lb, page, G, tile, fp8):
    wl = WL.random_decode(30 + page // 64, 7, 4000)
    wl.kv_lens[0] = 0
    wl.kv_lens[1] = page + 1                      # one token into a second page
    wl.kv_lens[-1] = max(wl.kv_lens[-1], 2 * page + 70)
    note(f"decode page={page} G={G} tile={tile} fp8={fp8} lens={wl.kv_lens}")
    words = lb.attn_plan(wl.kv_lens, 9, tile)
    assert np.array_equal(words, ref_plan(wl.kv_lens, 9, tile))
    if fp8:
        inputs = decode_inputs_fp8(wl, page=page, pad_code=NAN_CODE)
        ref = oracle_decode_fp8(wl)
    else:
        inputs = decode_inputs(wl, page=page, pad_value=float("nan"))
        ref = oracle_decode(wl)
    got = _decode(lb, wl, words, inputs, G, fp8)
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"page {page} request {b} (L={wl.kv_lens[b]})")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("page", [128, 256])
def test_mtp_page_sizes(lb, page, fp8):
    from load_balanced_split_attn_amd.mtp import MtpDecodeStep
    wl = WL.random_mtp(40 + page // 64, 6, 3000)
    wl.q_lens[-1] = 4
    wl.kv_lens[0] = max(wl.kv_lens[0], page + 3)
    note(f"mtp page={page} fp8={fp8} kv={wl.kv_lens} q={wl.q_lens}")
    q, kc, vc, bt, scales = mtp_inputs(wl, page=page, fp8=fp8, pad=NAN_CODE if fp8 else float("nan"))
    step = MtpDecodeStep(wl.q_lens, wl.kv_lens, q.device, num_workers=11, head_groups=8,
                         kv_dtype=lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16)
    assert np.array_equal(step.map_host, ref_plan_prefill(wl.q_lens, wl.kv_lens, 11, step.R, 512, True))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out, kv_scales=scales)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    starts = q_starts(wl)
    for b, r in oracle_mtp(wl, fp8=fp8).items():
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], r, f"page {page} request {b}")


@pytest.mark.parametrize("exact_pv", [None, False, True])
@pytest.mark.parametrize("page", [128, 256])
def test_prefill_page_sizes(page, exact_pv):
    from load_balanced_split_attn_amd.prefill import PrefillStep
    wl = WL.random_prefill(50 + page // 64, 3, 1500, 300)
    note(f"prefill page={page} exact_pv={exact_pv} q={wl.q_lens} kv={wl.kv_lens}")
    q, kc, vc, bt = prefill_inputs(wl, page=page, pad_value=float("nan"))
    step = PrefillStep(wl.q_lens, wl.kv_lens, q.device, num_workers=5, exact_pv=exact_pv)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    starts = q_starts(wl)
    for b in range(wl.batch):
        k, v = wl.kv(b)
        ref = ref_attention(wl.q(b).double().numpy(), k.double().numpy(), v.double().numpy(), SCALE, causal=True)
        assert_close(got[starts[b]:starts[b] + wl.q_lens[b]], ref, f"page {page} request {b}")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("page", [128, 1024])
def test_store_kv_page_sizes(lb, page, fp8):
    """The producer step appends at every offset class of a larger page (first token, inside the
    first 32/64-token tile, past it, last token); the stored values read back in place."""
    from load_balanced_split_attn_amd.paged import cache_shapes, unpack_request
    from oracle import store_kv as SK
    dev = torch.device("cuda")
    lens = [0, 31, 64, 100, page - 1, page, 2 * page - 1]
    B = len(lens)
    g = torch.Generator().manual_seed(page + fp8)
    q = torch.randn(B, 64, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(B, 8, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, 8, 128, generator=g).to(torch.bfloat16)
    need = [L // page + 1 for L in lens]
    P = sum(need)
    dtype = torch.uint8 if fp8 else torch.bfloat16
    ksh, vsh = cache_shapes(P, 8, page, 128, dtype)
    kc = torch.zeros(ksh, dtype=dtype, device=dev)
    vc = torch.zeros(vsh, dtype=dtype, device=dev)
    bt = torch.zeros((B, max(need)), dtype=torch.int32)
    first = 0
    for b, n in enumerate(need):
        bt[b, :n] = torch.arange(first, first + n, dtype=torch.int32).flip(0)   # pages in reverse
        first += n
    bt = bt.to(dev)
    scales = None
    if fp8:
        scales = (torch.full((8,), 0.03, device=dev), torch.full((8,), 0.02, device=dev))
    q_out = torch.empty_like(q, device=dev)
    lb.attn_store_kv(q.to(dev), k.to(dev), v.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev), q_out,
                     kc, vc, bt, rope_theta=10000.0, hadamard=True, kv_scales=scales)
    torch.cuda.synchronize()
    _, rk, rv = SK.ref_store_kv(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                np.array(lens, dtype=np.float64), None, None, 1e-6, 10000.0, True,
                                np.full(8, 0.03) if fp8 else None, np.full(8, 0.02) if fp8 else None)
    for b, L in enumerate(lens):
        kb, vb = unpack_request(kc, vc, bt, b, L + 1)
        for got, ref in ((kb[L].cpu(), rk[b]), (vb[L].cpu(), rv[b])):
            if fp8:
                # codes equal, or one code apart where fp32 and fp64 fall on different sides of a tie
                assert np.max(np.abs(got.numpy().astype(np.int32) - ref.astype(np.int32))) <= 1, f"page {page} b {b}"
                assert np.mean(got.numpy() == ref) > 0.98
            else:
                d = np.abs(got.double().numpy() - ref)
                assert np.all(d <= np.ldexp(1.0, np.frexp(ref)[1] - 8) + 1e-5 * np.max(np.abs(ref))), f"page {page} b {b}"
    # nothing but the B new tokens was written
    stored = sum(int(torch.count_nonzero(unpack_request(kc, vc, bt, b, L + 1)[0][L]).item()) for b, L in enumerate(lens))
    assert int(torch.count_nonzero(kc).item()) == stored


@pytest.mark.parametrize("fp8", [False, True])
def test_many_small_requests(lb, fp8):
    """777 requests of 0-130 tokens on the device's own worker count: most workers hold several
    requests, many requests hold no tile, and the combine covers 777 units."""
    wl = WL.random_decode(60 + int(fp8), 777, 130)
    W = lb.attn_query_workers(0, 8, lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16)
    note(f"many small requests fp8={fp8}: B={wl.batch} tokens={sum(wl.kv_lens)} zeros={wl.kv_lens.count(0)} W={W}")
    words = lb.attn_plan(wl.kv_lens, W, 512)
    assert np.array_equal(words, ref_plan(wl.kv_lens, W, 512))
    if fp8:
        got = _decode(lb, wl, words, decode_inputs_fp8(wl, pad_code=NAN_CODE), 8, True)
        ref = oracle_decode_fp8(wl)
    else:
        got = _decode(lb, wl, words, decode_inputs(wl, pad_value=float("nan")), 8, False)
        ref = oracle_decode(wl)
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"request {b} (L={wl.kv_lens[b]})")
