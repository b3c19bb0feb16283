"""attn_kv_layout: a paged cache in the token-major layout [P, Hkv, page, D] converted to the blocked
layout the attention kernels read and back, bit for bit against the layout's definition
(paged.to_blocked, element positions pinned on the CPU by test_paged_cpu.py), and a decode step over
a converted cache against the fp64 oracle."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import SCALE, assert_close, note, oracle_decode
from load_balanced_split_attn_amd.paged import to_blocked

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.uint8])
@pytest.mark.parametrize("page,P,Hkv", [(64, 37, 8), (256, 5, 2), (128, 1, 1)])
def test_round_trip_matches_definition(lb, dtype, page, P, Hkv):
    g = torch.Generator().manual_seed(page + P)
    elem = 2 if dtype == torch.bfloat16 else 1
    raw = lambda: torch.randint(0, 256, (P * page, Hkv, 128 * elem), generator=g, dtype=torch.uint8).view(dtype)
    k, v = raw(), raw()   # token-major rows [P * page, Hkv, D]
    tm_k = k.view(P, page, Hkv, 128).permute(0, 2, 1, 3).contiguous()
    tm_v = v.view(P, page, Hkv, 128).permute(0, 2, 1, 3).contiguous()
    kb_ref, vb_ref = to_blocked(k, v, page)
    dev = torch.device("cuda")
    note(f"layout {dtype} page={page} P={P} Hkv={Hkv}")
    kb = torch.full(kb_ref.shape, 0, dtype=dtype, device=dev)
    vb = torch.full(vb_ref.shape, 0, dtype=dtype, device=dev)
    lb.attn_kv_layout(tm_k.to(dev), tm_v.to(dev), kb, vb, to_blocked=True)
    back_k = torch.zeros(tm_k.shape, dtype=dtype, device=dev)
    back_v = torch.zeros(tm_v.shape, dtype=dtype, device=dev)
    lb.attn_kv_layout(kb, vb, back_k, back_v, to_blocked=False)
    torch.cuda.synchronize()
    assert torch.equal(kb.cpu().view(torch.uint8), kb_ref.contiguous().view(torch.uint8))
    assert torch.equal(vb.cpu().view(torch.uint8), vb_ref.contiguous().view(torch.uint8))
    assert torch.equal(back_k.cpu().view(torch.uint8), tm_k.view(torch.uint8))
    assert torch.equal(back_v.cpu().view(torch.uint8), tm_v.view(torch.uint8))


def test_refusals(lb):
    dev = torch.device("cuda")
    a = torch.zeros((2, 8, 64, 128), dtype=torch.bfloat16, device=dev)
    kb = torch.zeros((2, 8, 4, 64, 32), dtype=torch.bfloat16, device=dev)
    vb = torch.zeros((2, 8, 2, 128, 32), dtype=torch.bfloat16, device=dev)
    lib = lb.lib()
    p = lb._dptr
    assert lib.attn_kv_layout(p(a), p(a), p(kb), p(vb), 2, 8, 64, 128, 0, 2, None) == -1      # direction
    assert lib.attn_kv_layout(p(a), p(a), p(a), p(vb), 2, 8, 64, 128, 0, 0, None) == -1      # in place
    assert lib.attn_kv_layout(p(a), p(a), p(kb), p(vb), 2, 8, 96, 128, 0, 0, None) == -3     # page % 64
    assert lib.attn_kv_layout(p(a), p(a), p(kb), p(vb), 2, 8, 64, 64, 0, 0, None) == -3      # head dim
    assert lib.attn_kv_layout(p(a), p(a), p(kb), p(vb), 2, 8, 64, 128, 5, 0, None) == -1     # dtype


def test_decode_over_converted_cache(lb):
    """A token-major paged cache (shuffled pages) converted with attn_kv_layout, then a decode step:
    outputs against the fp64 oracle."""
    from load_balanced_split_attn_amd.decode import DecodeStep
    from load_balanced_split_attn_amd.paged import pages_for
    wl = WL.random_decode(71, 6, 3000, min_len=1)
    dev = torch.device("cuda")
    page, Hkv, D = 64, wl.hkv, wl.head_dim
    npages = [pages_for(L, page) for L in wl.kv_lens]
    P = sum(npages)
    perm = wl.page_permutation(P)
    tm_k = torch.zeros((P, Hkv, page, D), dtype=torch.bfloat16)
    tm_v = torch.zeros((P, Hkv, page, D), dtype=torch.bfloat16)
    bt = torch.zeros((wl.batch, max(npages)), dtype=torch.int32)
    first = 0
    for b, L in enumerate(wl.kv_lens):
        k, v = wl.kv(b)
        for lp in range(npages[b]):
            pid = int(perm[first + lp])
            bt[b, lp] = pid
            n = min(page, L - lp * page)
            tm_k[pid, :, :n] = k[lp * page:lp * page + n].permute(1, 0, 2)
            tm_v[pid, :, :n] = v[lp * page:lp * page + n].permute(1, 0, 2)
        first += npages[b]
    kc = torch.empty((P, Hkv, D // 32, page, 32), dtype=torch.bfloat16, device=dev)
    vc = torch.empty((P, Hkv, page // 32, D, 32), dtype=torch.bfloat16, device=dev)
    lb.attn_kv_layout(tm_k.to(dev), tm_v.to(dev), kc, vc)
    q = wl.q().to(dev)
    out = DecodeStep(wl.kv_lens, dev, num_workers=9)(q, kc, vc, bt.to(dev), scale=SCALE)
    torch.cuda.synchronize()
    ref = oracle_decode(wl)
    got = out.cpu().numpy()
    for b in range(wl.batch):
        assert_close(got[b], ref[b], f"request {b}")
