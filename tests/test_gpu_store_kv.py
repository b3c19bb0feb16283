"""GPU parity of the fused producer step (attn_store_kv) against the fp64 oracle: the rotated q,
the stored K/V (bf16 values or E4M3 codes) read back from the blocked paged cache, exact hardware
rounding where the input fixes it, and a decode step over the appended tokens end to end."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import SCALE, assert_close, note
from oracle import store_kv as SK
from oracle.attention import ref_attention
from oracle.fp8 import dequantize_kv, e4m3_table

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _bf16_step(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def _tol(ref):
    """One bf16 step at the value, plus the fp32 arithmetic's absolute error on a head vector (a
    128-term Hadamard sum): 1e-5 of the vector's largest magnitude.  Near-zero outputs have bf16
    steps far below that error, so their rounding may land one or more steps away."""
    ref = np.asarray(ref, dtype=np.float64)
    return _bf16_step(ref) + 1e-5 * np.max(np.abs(ref), axis=-1, keepdims=True)


def _inputs(seed, B, Hq=64, Hkv=8, D=128):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    k = (torch.randn(B, Hkv, D, generator=g) * 2).to(torch.bfloat16)
    v = torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16)
    qw = (1 + 0.3 * torch.randn(D, generator=g)).float()
    kw = (1 + 0.3 * torch.randn(D, generator=g)).float()
    return q, k, v, qw, kw


def _empty_cache(lens, page, fp8, dev, Hkv=8, D=128):
    """A paged cache holding len_b tokens per request plus room for one more; contents zero."""
    from load_balanced_split_attn_amd.paged import cache_shapes, pages_for
    need = [pages_for(L + 1, page) for L in lens]
    P = sum(need)
    dtype = torch.uint8 if fp8 else torch.bfloat16
    ks, vs = cache_shapes(P, Hkv, page, D, dtype)
    kc = torch.zeros(ks, dtype=dtype, device=dev)
    vc = torch.zeros(vs, dtype=dtype, device=dev)
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(3))
    bt = torch.zeros((len(lens), max(need)), dtype=torch.int32)
    first = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[first:first + n].to(torch.int32)
        first += n
    return kc, vc, bt.to(dev)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("norm,theta,had", [(True, 10000.0, True), (False, 1e6, False), (True, 0.0, True),
                                            (False, 0.0, False)])
def test_store_matches_oracle(lb, fp8, norm, theta, had):
    from load_balanced_split_attn_amd.paged import unpack_request
    dev = torch.device("cuda")
    B = 37
    q, k, v, qw, kw = _inputs(40 + int(fp8), B)
    lens = [int(x) for x in np.random.default_rng(7).integers(0, 200000, size=B)]
    lens[0], lens[1] = 0, 63                      # first token of a page, last token of a page
    kc, vc, bt = _empty_cache(lens, 64, fp8, dev)
    pos = torch.tensor(lens, dtype=torch.int32, device=dev)
    ks = vs = None
    if fp8:
        ks = torch.exp2(torch.rand(8, generator=torch.Generator().manual_seed(9)) * 2 - 5).float()
        vs = torch.exp2(torch.rand(8, generator=torch.Generator().manual_seed(10)) * 2 - 6).float()
    q_out = torch.empty_like(q, device=dev)
    lb.attn_store_kv(q.to(dev), k.to(dev), v.to(dev), pos, q_out, kc, vc, bt,
                     q_norm_w=qw.to(dev) if norm else None, k_norm_w=kw.to(dev) if norm else None, eps=1e-6,
                     rope_theta=theta, hadamard=had, kv_scales=(ks.to(dev), vs.to(dev)) if fp8 else None)
    torch.cuda.synchronize()
    rq, rk, rv = SK.ref_store_kv(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                 np.array(lens, dtype=np.float64), qw.double().numpy() if norm else None,
                                 kw.double().numpy() if norm else None, 1e-6, theta, had,
                                 ks.double().numpy() if fp8 else None, vs.double().numpy() if fp8 else None)
    got_q = q_out.float().cpu().numpy().astype(np.float64)
    dq = np.abs(got_q - rq)
    assert np.all(dq <= _tol(rq)), f"q: {int((dq > _tol(rq)).sum())} beyond tolerance"
    assert np.mean(dq == 0) > 0.99
    table = e4m3_table()
    for b, L in enumerate(lens):
        kb, vb = unpack_request(kc, vc, bt, b, L + 1)
        got_k, got_v = kb[L].cpu(), vb[L].cpu()
        if fp8:
            gk, gv = got_k.numpy(), got_v.numpy()
            for got, ref, sc in ((gk, rk[b], ks), (gv, rv[b], vs)):
                # codes equal, or one step apart where fp32 and fp64 land on different sides of a tie
                dv = np.abs(table[got] - table[ref])
                step = np.abs(table[np.minimum(ref.astype(np.int32) & 0x7F, 0x7D) + 1] - table[ref.astype(np.int32) & 0x7F])
                assert np.all((got == ref) | (dv <= step + 1e-12)), f"request {b}"
                assert np.mean(got == ref) > 0.98
        else:
            for got, ref in ((got_k.double().numpy(), rk[b]), (got_v.double().numpy(), rv[b])):
                assert np.all(np.abs(got - ref) <= _tol(ref)), f"request {b}"
    note(f"fp8={fp8} norm={norm} theta={theta} hadamard={had}: q exact {np.mean(dq == 0):.4f}")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("hq,hkv", [(6, 3), (5, 1), (12, 4)])
def test_store_head_counts(lb, fp8, hq, hkv):
    """Head counts that leave rows of a wave without a head (a wave holds four head vectors of one
    kind): every stored value still matches the oracle and nothing past the heads is written."""
    from load_balanced_split_attn_amd.paged import unpack_request
    dev = torch.device("cuda")
    B = 9
    q, k, v, qw, kw = _inputs(90 + hq, B, Hq=hq, Hkv=hkv)
    lens = [int(x) for x in np.random.default_rng(hq).integers(0, 3000, size=B)]
    kc, vc, bt = _empty_cache(lens, 64, fp8, dev, Hkv=hkv)
    pos = torch.tensor(lens, dtype=torch.int32, device=dev)
    ks = vs = None
    if fp8:
        ks = torch.exp2(torch.rand(hkv, generator=torch.Generator().manual_seed(11)) * 2 - 5).float()
        vs = torch.exp2(torch.rand(hkv, generator=torch.Generator().manual_seed(12)) * 2 - 6).float()
    q_dev = q.to(dev)
    q_out = torch.full((B + 1, hq, 128), 7.0, dtype=torch.bfloat16, device=dev)   # one row of guard
    lb.attn_store_kv(q_dev, k.to(dev), v.to(dev), pos, q_out[:B], kc, vc, bt, q_norm_w=qw.to(dev),
                     k_norm_w=kw.to(dev), rope_theta=10000.0, hadamard=True,
                     kv_scales=(ks.to(dev), vs.to(dev)) if fp8 else None)
    torch.cuda.synchronize()
    assert torch.all(q_out[B] == 7.0)
    rq, rk, rv = SK.ref_store_kv(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                 np.array(lens, dtype=np.float64), qw.double().numpy(), kw.double().numpy(),
                                 1e-6, 10000.0, True, ks.double().numpy() if fp8 else None,
                                 vs.double().numpy() if fp8 else None)
    dq = np.abs(q_out[:B].float().cpu().numpy().astype(np.float64) - rq)
    assert np.all(dq <= _tol(rq))
    table = e4m3_table()
    for b, L in enumerate(lens):
        kb, vb = unpack_request(kc, vc, bt, b, L + 1)
        for got, ref in ((kb[L].cpu(), rk[b]), (vb[L].cpu(), rv[b])):
            if fp8:
                g = got.numpy()
                dv = np.abs(table[g] - table[ref])
                step = np.abs(table[np.minimum(ref.astype(np.int32) & 0x7F, 0x7D) + 1] - table[ref.astype(np.int32) & 0x7F])
                assert np.all((g == ref) | (dv <= step + 1e-12)), f"request {b}"
            else:
                assert np.all(np.abs(got.double().numpy() - ref) <= _tol(ref)), f"request {b}"
    # exactly the B new tokens were written: nonzero elements only at the stored positions, K and V
    for which, cache in ((0, kc), (1, vc)):
        stored = sum(int(torch.count_nonzero(unpack_request(kc, vc, bt, b, L + 1)[which][L]).item())
                     for b, L in enumerate(lens))
        assert int(torch.count_nonzero(cache).item()) == stored, "KV"[which] + " cache: stray writes"


def test_hardware_rounding_exact(lb):
    """With no norm, RoPE or Hadamard the stored V is the input itself: the bf16 path stores it
    unchanged and the E4M3 path rounds x / scale with scale 1 exactly as the oracle does, exact
    midpoints between neighbouring codes included (ties to even)."""
    from load_balanced_split_attn_amd.paged import unpack_request
    dev = torch.device("cuda")
    table = e4m3_table()
    vals = table[np.arange(0, 0x7F)]
    mids = (vals[:-1] + vals[1:]) / 2
    cand = np.concatenate([mids, -mids, vals, -vals, [500.0, -1000.0, 1e-4, -1e-4]])
    cand = torch.from_numpy(cand).to(torch.bfloat16)
    keep = cand.double().numpy()
    B = -(-len(keep) // (8 * 128))
    v = torch.zeros(B * 8 * 128, dtype=torch.bfloat16)
    v[:len(keep)] = cand
    v = v.view(B, 8, 128)
    q, k, _, _, _ = _inputs(50, B)
    lens = [5] * B
    pos = torch.tensor(lens, dtype=torch.int32, device=dev)
    for fp8 in (False, True):
        kc, vc, bt = _empty_cache(lens, 64, fp8, dev)
        ones = torch.ones(8, dtype=torch.float32, device=dev)
        q_out = torch.empty_like(q, device=dev)
        lb.attn_store_kv(q.to(dev), k.to(dev), v.to(dev), pos, q_out, kc, vc, bt,
                         kv_scales=(ones, ones) if fp8 else None)
        torch.cuda.synchronize()
        got = torch.cat([unpack_request(kc, vc, bt, b, 6)[1][5].reshape(-1).cpu() for b in range(B)])
        ref = v.reshape(-1).double().numpy()
        if fp8:
            assert np.array_equal(got.numpy(), SK.e4m3_round(np.clip(ref, -448, 448)))
        else:
            assert np.array_equal(got.double().numpy(), ref)
        assert torch.equal(q_out.cpu(), q)                # q unchanged when every step is off


def test_out_of_table_positions_not_stored(lb):
    dev = torch.device("cuda")
    q, k, v, _, _ = _inputs(60, 3)
    kc, vc, bt = _empty_cache([10, 20, 30], 64, False, dev)
    pos = torch.tensor([10, 5000, -1], dtype=torch.int32, device=dev)
    q_out = torch.empty_like(q, device=dev)
    lb.attn_store_kv(q.to(dev), k.to(dev), v.to(dev), pos, q_out, kc, vc, bt)
    torch.cuda.synchronize()
    from load_balanced_split_attn_amd.paged import unpack_request
    kb, vb = unpack_request(kc, vc, bt, 0, 11)
    assert torch.equal(kb[10].cpu(), k[0])
    assert torch.equal(vb[10].cpu(), v[0])
    # nothing else was written, in either cache
    assert int(torch.count_nonzero(kc).item()) == int(torch.count_nonzero(k[0]).item())
    assert int(torch.count_nonzero(vc).item()) == int(torch.count_nonzero(v[0]).item())


@pytest.mark.parametrize("fp8", [False, True])
def test_append_then_decode(lb, fp8):
    """A decode step end to end: each request's cache holds L_b tokens; the producer step appends the
    new token (RMSNorm + RoPE + Hadamard on q and k), then decode attention runs over L_b + 1 keys
    with the produced q.  Reference: the oracle's stored values and rotated q, plain attention."""
    from load_balanced_split_attn_amd.decode import DecodeStep
    from load_balanced_split_attn_amd.paged import pack_paged
    dev = torch.device("cuda")
    wl = WL.random_decode(70 + int(fp8), 6, 3000, min_len=1)
    B = wl.batch
    q, k, v, qw, kw = _inputs(80, B)
    # caches with room for the new token: pack L_b + 1 tokens whose last one is a placeholder
    ks = vs = None
    if fp8:
        ks, vs = wl.kv_scales()
        old = [wl.kv_fp8(b) for b in range(B)]
        kv_of = lambda b: (torch.cat([old[b][0], torch.zeros(1, 8, 128, dtype=torch.uint8)]),
                           torch.cat([old[b][1], torch.zeros(1, 8, 128, dtype=torch.uint8)]))
    else:
        old = [wl.kv(b) for b in range(B)]
        kv_of = lambda b: (torch.cat([old[b][0], torch.zeros(1, 8, 128, dtype=torch.bfloat16)]),
                           torch.cat([old[b][1], torch.zeros(1, 8, 128, dtype=torch.bfloat16)]))
    new_lens = [L + 1 for L in wl.kv_lens]
    kc, vc, bt = pack_paged(kv_of, new_lens, 64, 8, 128, wl.page_permutation, dev,
                            dtype=torch.uint8 if fp8 else torch.bfloat16)
    pos = torch.tensor(wl.kv_lens, dtype=torch.int32, device=dev)
    q_out = torch.empty_like(q, device=dev)
    scales = (ks.to(dev), vs.to(dev)) if fp8 else None
    lb.attn_store_kv(q.to(dev), k.to(dev), v.to(dev), pos, q_out, kc, vc, bt, q_norm_w=qw.to(dev),
                     k_norm_w=kw.to(dev), rope_theta=10000.0, hadamard=True, kv_scales=scales)
    step = DecodeStep(new_lens, dev, num_workers=11, kv_dtype=lb.KV_FP8_E4M3 if fp8 else lb.KV_BF16)
    out = step(q_out, kc, vc, bt, scale=SCALE, kv_scales=scales)
    torch.cuda.synchronize()
    rq, rk, rv = SK.ref_store_kv(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                 np.array(wl.kv_lens, dtype=np.float64), qw.double().numpy(), kw.double().numpy(),
                                 1e-6, 10000.0, True, ks.double().numpy() if fp8 else None,
                                 vs.double().numpy() if fp8 else None)
    got = out.cpu().numpy()
    qg = q_out.float().cpu().numpy().astype(np.float64)   # attention parity against the produced q
    for b in range(B):
        if fp8:
            kk = dequantize_kv(np.concatenate([old[b][0].numpy(), rk[b:b + 1]]), ks.double().numpy())
            vv = dequantize_kv(np.concatenate([old[b][1].numpy(), rv[b:b + 1]]), vs.double().numpy())
        else:
            kk = np.concatenate([old[b][0].double().numpy(), rk[b:b + 1]])
            vv = np.concatenate([old[b][1].double().numpy(), rv[b:b + 1]])
        ref = ref_attention(qg[b:b + 1], kk, vv, SCALE)[0]
        assert_close(got[b], ref, f"append+decode fp8={fp8} request {b}")


@pytest.mark.parametrize("seed", range(96))
def test_store_random_sweep(lb, seed):
    """Seeded random producer steps crossing what the cases above take one at a time: batch size,
    head counts, page size, 8-bit or bf16 cache, RMSNorm on or off, RoPE base (0 = off), Hadamard
    on or off, eps and positions; q against the oracle with a guard row, every stored K/V value,
    and nothing written outside the stored positions."""
    from load_balanced_split_attn_amd.paged import unpack_request
    g = np.random.default_rng([7, seed])
    dev = torch.device("cuda")
    max_pos = int(g.choice([100, 5000, 200000]))
    B = int(g.integers(1, 300 if max_pos <= 5000 else 12))    # cache kept to a few GB
    hq, hkv = [(64, 8), (8, 1), (6, 3), (12, 4), (16, 2), (32, 8)][int(g.integers(0, 6))]
    page = int(g.choice([64, 128, 256]))
    fp8 = bool(g.random() < 0.5)
    norm = bool(g.random() < 0.5)
    theta = float(g.choice([0.0, 10000.0, 1e6]))
    had = bool(g.random() < 0.5)
    eps = float(g.choice([1e-6, 1e-5]))
    note(f"store sweep {seed}: B={B} heads={hq}/{hkv} page={page} fp8={fp8} norm={norm} theta={theta} "
         f"hadamard={had} max_pos={max_pos}")
    q, k, v, qw, kw = _inputs(500 + seed, B, Hq=hq, Hkv=hkv)
    lens = [int(x) for x in g.integers(0, max_pos, size=B)]
    kc, vc, bt = _empty_cache(lens, page, fp8, dev, Hkv=hkv)
    pos = torch.tensor(lens, dtype=torch.int32, device=dev)
    ks = vs = None
    if fp8:
        ks = torch.exp2(torch.rand(hkv, generator=torch.Generator().manual_seed(20 + seed)) * 2 - 5).float()
        vs = torch.exp2(torch.rand(hkv, generator=torch.Generator().manual_seed(40 + seed)) * 2 - 6).float()
    q_out = torch.full((B + 1, hq, 128), 7.0, dtype=torch.bfloat16, device=dev)   # one row of guard
    lb.attn_store_kv(q.to(dev), k.to(dev), v.to(dev), pos, q_out[:B], kc, vc, bt,
                     q_norm_w=qw.to(dev) if norm else None, k_norm_w=kw.to(dev) if norm else None, eps=eps,
                     rope_theta=theta, hadamard=had, kv_scales=(ks.to(dev), vs.to(dev)) if fp8 else None)
    torch.cuda.synchronize()
    assert torch.all(q_out[B] == 7.0)
    rq, rk, rv = SK.ref_store_kv(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                 np.array(lens, dtype=np.float64), qw.double().numpy() if norm else None,
                                 kw.double().numpy() if norm else None, eps, theta, had,
                                 ks.double().numpy() if fp8 else None, vs.double().numpy() if fp8 else None)
    dq = np.abs(q_out[:B].float().cpu().numpy().astype(np.float64) - rq)
    assert np.all(dq <= _tol(rq)), f"q: {int((dq > _tol(rq)).sum())} beyond tolerance"
    table = e4m3_table()
    for b, L in enumerate(lens):
        kb, vb = unpack_request(kc, vc, bt, b, L + 1)
        for got, ref in ((kb[L].cpu(), rk[b]), (vb[L].cpu(), rv[b])):
            if fp8:
                gc = got.numpy()
                dv = np.abs(table[gc] - table[ref])
                step = np.abs(table[np.minimum(ref.astype(np.int32) & 0x7F, 0x7D) + 1] - table[ref.astype(np.int32) & 0x7F])
                assert np.all((gc == ref) | (dv <= step + 1e-12)), f"request {b}"
            else:
                assert np.all(np.abs(got.double().numpy() - ref) <= _tol(ref)), f"request {b}"
    for which, cache in ((0, kc), (1, vc)):
        stored = sum(int(torch.count_nonzero(unpack_request(kc, vc, bt, b, L + 1)[which][L]).item())
                     for b, L in enumerate(lens))
        written = sum(int(torch.count_nonzero(cache[p0:p0 + 256]).item()) for p0 in range(0, cache.shape[0], 256))
        assert written == stored, "KV"[which] + " cache: stray writes"


def _prefilled_cache(totals, page, fp8, dev, seed, Hkv=8, D=128):
    """A paged cache whose every slot (tokens, and pads up to the page end) holds random bytes, so
    that a write outside the intended tokens shows; seeded page permutation."""
    from load_balanced_split_attn_amd.paged import pack_paged
    g = torch.Generator().manual_seed(seed)
    dtype = torch.uint8 if fp8 else torch.bfloat16

    def kv_of(b):
        L = totals[b]
        if fp8:
            return (torch.randint(0, 256, (L, Hkv, D), generator=g, dtype=torch.uint8),
                    torch.randint(0, 256, (L, Hkv, D), generator=g, dtype=torch.uint8))
        return (torch.randn(L, Hkv, D, generator=g).to(torch.bfloat16), torch.randn(L, Hkv, D, generator=g).to(torch.bfloat16))

    perm = lambda n: torch.randperm(n, generator=torch.Generator().manual_seed(seed + 1))
    return pack_paged(kv_of, totals, page, Hkv, D, perm, dev, pad_value=77 if fp8 else 3.5, dtype=dtype)


@pytest.mark.parametrize("page", [64, 256])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("norm,theta,had", [(True, 10000.0, True), (False, 0.0, False)])
def test_chunk_append(lb, fp8, norm, theta, had, page):
    """attn_store_kv_chunk (chunked-prefill append: V written in whole 64-byte rows) stores exactly
    what the one-token path stores for the same tokens, leaves every other byte of the cache as it
    was (the prefix before each chunk and the slots after it share rows with the chunk's first and
    last tokens), writes the same rotated q, and matches the fp64 oracle.  Chunks start on and off
    row boundaries, span one token to several pages, and one request appends nothing."""
    _check_chunk_append(lb, fp8, norm, theta, had, page)


@pytest.mark.parametrize("hq,hkv", [(8, 1), (6, 3), (12, 4), (20, 2), (32, 8), (68, 12)])
@pytest.mark.parametrize("fp8", [False, True])
def test_chunk_append_head_counts(lb, fp8, hq, hkv):
    """The chunk append's q/k workgroups loop over four-head tasks per wave with the next task's
    loads in flight: head counts that leave a wave without a task or give it one to five (some with
    rows past the last head), bitwise the one-token path and against the oracle, as above."""
    _check_chunk_append(lb, fp8, True, 10000.0, True, 64, hq=hq, hkv=hkv)


def _check_chunk_append(lb, fp8, norm, theta, had, page, hq=64, hkv=8):
    from load_balanced_split_attn_amd.paged import unpack_request
    dev = torch.device("cuda")
    prefix = [0, 31, 64, 100, 1000, 5, 4096]
    n = [300, 1, 64, 0, 129, 2000, 33]
    extra = [5, 0, 40, 7, 100, 3, 90]
    totals = [p + c + e for p, c, e in zip(prefix, n, extra)]
    B, rows = len(n), sum(n)
    note(f"chunk append fp8={fp8} norm={norm} theta={theta} had={had} page={page} heads={hq}/{hkv}")
    kc0, vc0, bt = _prefilled_cache(totals, page, fp8, dev, seed=90 + int(fp8), Hkv=hkv)
    q, k, v, qw, kw = _inputs(80 + int(fp8), rows, Hq=hq, Hkv=hkv)
    starts = np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int32)
    q_lens = torch.tensor(n, dtype=torch.int32, device=dev)
    q_start = torch.tensor(starts, dtype=torch.int32, device=dev)
    pos0 = torch.tensor(prefix, dtype=torch.int32, device=dev)
    ks = vs = None
    if fp8:
        ks = torch.tensor([0.02 * (1 + 0.1 * h) for h in range(hkv)], dtype=torch.float32, device=dev)
        vs = torch.tensor([0.03 * (1 + 0.05 * h) for h in range(hkv)], dtype=torch.float32, device=dev)
    kw_args = dict(q_norm_w=qw.to(dev) if norm else None, k_norm_w=kw.to(dev) if norm else None, eps=1e-6,
                   rope_theta=theta, hadamard=had, kv_scales=(ks, vs) if fp8 else None)
    kc1, vc1 = kc0.clone(), vc0.clone()
    q1 = torch.full((rows, hq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lb.attn_store_kv_chunk(q.to(dev), k.to(dev), v.to(dev), q_lens, q_start, pos0, max(n), q1, kc1, vc1, bt, **kw_args)
    # the one-token path over the same rows: row r of request b at position prefix[b] + j
    req = np.repeat(np.arange(B), n)
    pos_rows = torch.tensor([prefix[b] + j for b in range(B) for j in range(n[b])], dtype=torch.int32, device=dev)
    bt_rows = bt[torch.from_numpy(req).to(dev)].contiguous()
    kc2, vc2 = kc0.clone(), vc0.clone()
    q2 = torch.full((rows, hq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lb.attn_store_kv(q.to(dev), k.to(dev), v.to(dev), pos_rows, q2, kc2, vc2, bt_rows, **kw_args)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2), "rotated q differs from the one-token path"
    assert torch.equal(kc1, kc2), "K cache differs from the one-token path"
    assert torch.equal(vc1, vc2), "V cache differs from the one-token path"
    # every byte outside the chunks is the prefilled one
    for b in range(B):
        end = -(-totals[b] // page) * page
        k_new, v_new = unpack_request(kc1, vc1, bt, b, end)
        k_old, v_old = unpack_request(kc0, vc0, bt, b, end)
        keep = torch.ones(end, dtype=torch.bool)
        keep[prefix[b]:prefix[b] + n[b]] = False
        assert torch.equal(k_new[keep], k_old[keep]) and torch.equal(v_new[keep], v_old[keep]), f"request {b}: stray writes"
    # the stored values and q against the oracle
    rq, rk, rv = SK.ref_store_kv(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                 pos_rows.cpu().double().numpy(), qw.double().numpy() if norm else None,
                                 kw.double().numpy() if norm else None, 1e-6, theta, had,
                                 ks.cpu().double().numpy() if fp8 else None, vs.cpu().double().numpy() if fp8 else None)
    dq = np.abs(q1.float().cpu().numpy().astype(np.float64) - rq)
    assert np.all(dq <= _tol(rq)), f"q: {int((dq > _tol(rq)).sum())} beyond tolerance"
    table = e4m3_table()
    for b in range(B):
        if n[b] == 0:
            continue
        kb, vb = unpack_request(kc1, vc1, bt, b, prefix[b] + n[b])
        r0 = int(starts[b])
        for got, ref in ((kb[prefix[b]:].cpu(), rk[r0:r0 + n[b]]), (vb[prefix[b]:].cpu(), rv[r0:r0 + n[b]])):
            if fp8:
                gc = got.numpy()
                dv = np.abs(table[gc] - table[ref])
                step = np.abs(table[np.minimum(ref.astype(np.int32) & 0x7F, 0x7D) + 1] - table[ref.astype(np.int32) & 0x7F])
                assert np.all((gc == ref) | (dv <= step + 1e-12)), f"request {b}"
            else:
                assert np.all(np.abs(got.double().numpy() - ref) <= _tol(ref)), f"request {b}"


@pytest.mark.parametrize("seed", range(32))
def test_chunk_random_sweep(lb, seed):
    """Seeded random chunk appends crossing what the cases above take one at a time: batch size,
    prefix and chunk lengths (empty chunks included), a max_q_len above the longest chunk, a request
    with a negative start position (q written, nothing stored), head counts, page size, cache type,
    RMSNorm, RoPE base, Hadamard and eps.  q_out and both caches (prefilled with random bytes) bit
    for bit against the one-token path over the same tokens, and q against the fp64 oracle."""
    g = np.random.default_rng([11, seed])
    dev = torch.device("cuda")
    B = int(g.integers(1, 7))
    hq, hkv = [(64, 8), (8, 1), (6, 3), (12, 4), (16, 2), (32, 8), (68, 12)][int(g.integers(0, 7))]
    page = int(g.choice([64, 128, 256]))
    fp8 = bool(g.random() < 0.5)
    norm = bool(g.random() < 0.5)
    theta = float(g.choice([0.0, 10000.0, 1e6]))
    had = bool(g.random() < 0.5)
    eps = float(g.choice([1e-6, 1e-5]))
    prefix = [int(x) for x in g.integers(0, 3000, size=B)]
    n = [int(x) for x in g.integers(0, 300, size=B)]
    n[int(g.integers(0, B))] = int(g.integers(1, 300))
    extra = [int(x) for x in g.integers(0, 100, size=B)]
    neg = int(g.integers(0, B)) if g.random() < 0.2 else -1
    max_q = max(n) + int(g.integers(0, 3))
    note(f"chunk sweep {seed}: B={B} heads={hq}/{hkv} page={page} fp8={fp8} norm={norm} theta={theta} "
         f"hadamard={had} n={n} prefix={prefix} negative={neg}")
    totals = [p_ + c + e for p_, c, e in zip(prefix, n, extra)]
    rows = sum(n)
    kc0, vc0, bt = _prefilled_cache(totals, page, fp8, dev, seed=300 + seed, Hkv=hkv)
    q, k, v, qw, kw = _inputs(700 + seed, rows, Hq=hq, Hkv=hkv)
    starts = np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int32)
    pos_list = [(-1 - p_ if b == neg else p_) for b, p_ in enumerate(prefix)]
    q_lens = torch.tensor(n, dtype=torch.int32, device=dev)
    q_start = torch.tensor(starts, dtype=torch.int32, device=dev)
    pos0 = torch.tensor(pos_list, dtype=torch.int32, device=dev)
    ks = vs = None
    if fp8:
        ks = torch.exp2(torch.rand(hkv, generator=torch.Generator().manual_seed(50 + seed)) * 2 - 5).float().to(dev)
        vs = torch.exp2(torch.rand(hkv, generator=torch.Generator().manual_seed(60 + seed)) * 2 - 6).float().to(dev)
    kw_args = dict(q_norm_w=qw.to(dev) if norm else None, k_norm_w=kw.to(dev) if norm else None, eps=eps,
                   rope_theta=theta, hadamard=had, kv_scales=(ks, vs) if fp8 else None)
    kc1, vc1 = kc0.clone(), vc0.clone()
    q1 = torch.full((rows, hq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lb.attn_store_kv_chunk(q.to(dev), k.to(dev), v.to(dev), q_lens, q_start, pos0, max_q, q1, kc1, vc1, bt, **kw_args)
    # the one-token path: row j of request b at position pos_list[b] + j (all negative for the
    # request that starts below zero, so none of its tokens is stored)
    req = np.repeat(np.arange(B), n)
    pos_rows_l = [(pos_list[b] + j if pos_list[b] >= 0 else -1) for b in range(B) for j in range(n[b])]
    pos_rows = torch.tensor(pos_rows_l, dtype=torch.int32, device=dev)
    bt_rows = bt[torch.from_numpy(req).to(dev)].contiguous()
    kc2, vc2 = kc0.clone(), vc0.clone()
    q2 = torch.full((rows, hq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lb.attn_store_kv(q.to(dev), k.to(dev), v.to(dev), pos_rows, q2, kc2, vc2, bt_rows, **kw_args)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2), "rotated q differs from the one-token path"
    assert torch.equal(kc1, kc2), "K cache differs from the one-token path"
    assert torch.equal(vc1, vc2), "V cache differs from the one-token path"
    # q against the oracle at the positions the rows were rotated by: a request that starts below
    # zero takes position -1 for every row, as the one-token path does for a token at -1
    qpos = np.array(pos_rows_l, dtype=np.float64)
    rq, _, _ = SK.ref_store_kv(q.double().numpy(), k.double().numpy(), v.double().numpy(), qpos,
                               qw.double().numpy() if norm else None, kw.double().numpy() if norm else None,
                               eps, theta, had, ks.cpu().double().numpy() if fp8 else None,
                               vs.cpu().double().numpy() if fp8 else None)
    dq = np.abs(q1.float().cpu().numpy().astype(np.float64) - rq)
    assert np.all(dq <= _tol(rq)), f"q: {int((dq > _tol(rq)).sum())} beyond tolerance"


@pytest.mark.parametrize("fp8", [False, True])
def test_graph_captured_store(lb, fp8):
    """The producer step captured in a HIP graph: four replays with new q/k/v values and new
    positions written in place between them, and the program's own eager work in between; after
    every replay q_out and both caches equal, byte for byte, what the eager step writes into a copy of
    the caches taken before the replay."""
    lens = [37, 300, 1, 129, 64]
    dev = torch.device("cuda")
    B = len(lens)
    q, k, v, qw, kw = (t.to(dev) for t in _inputs(91, B))
    kc, vc, bt = _empty_cache([L + 3 for L in lens], 64, fp8, dev)
    scales = (torch.full((8,), 0.75, device=dev), torch.full((8,), 1.5, device=dev)) if fp8 else None
    pos = torch.tensor(lens, dtype=torch.int32, device=dev)
    q_out = torch.empty_like(q)
    args = dict(q_norm_w=qw, k_norm_w=kw, rope_theta=10000.0, hadamard=True, kv_scales=scales)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                           # warm-up outside the capture
        lb.attn_store_kv(q, k, v, pos, q_out, kc, vc, bt, **args)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lb.attn_store_kv(q, k, v, pos, q_out, kc, vc, bt, **args)
    torch.cuda.synchronize()
    for replay in range(4):
        nq, nk, nv, _, _ = (t.to(dev) for t in _inputs(200 + replay, B))
        q.copy_(nq), k.copy_(nk), v.copy_(nv)
        pos.copy_(torch.tensor([L + replay % 3 for L in lens], dtype=torch.int32))
        kc_e, vc_e, qo_e = kc.clone(), vc.clone(), torch.empty_like(q_out)
        lb.attn_store_kv(q, k, v, pos, qo_e, kc_e, vc_e, bt, **args)
        junk = torch.randn(1 << 16, device=dev).sum()   # the program's own eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(q_out, qo_e), f"replay {replay}: q_out"
        assert torch.equal(kc, kc_e) and torch.equal(vc, vc_e), f"replay {replay}: caches"
