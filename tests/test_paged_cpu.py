"""The blocked paged-cache layout (CPU only): element positions and the round trip through
pack_paged / unpack_request, for bf16 and 8-bit caches."""

import pytest
import torch

from load_balanced_split_attn_amd.paged import cache_shapes, pack_paged, unpack_request


@pytest.mark.parametrize("dtype,w", [(torch.bfloat16, 32), (torch.uint8, 64)])
@pytest.mark.parametrize("page", [64, 128])
def test_blocked_layout_positions_and_round_trip(dtype, w, page):
    g = torch.Generator().manual_seed(3)
    lens = [1, page + 5, 3 * page, 0, 2 * page - 1]
    Hkv, D = 4, 128

    def draw(L):
        x = torch.randint(0, 250, (L, Hkv, D), generator=g, dtype=torch.int32)
        return x.to(dtype)

    kvs = [(draw(L), draw(L)) for L in lens]
    perm = lambda n: torch.randperm(n, generator=torch.Generator().manual_seed(7))
    kc, vc, bt = pack_paged(lambda b: kvs[b], lens, page, Hkv, D, perm, "cpu", pad_value=0, dtype=dtype)
    P = kc.shape[0]
    assert (tuple(kc.shape), tuple(vc.shape)) == cache_shapes(P, Hkv, page, D, dtype)
    flat_k = kc.reshape(P, Hkv, -1)
    flat_v = vc.reshape(P, Hkv, -1)
    for b, L in enumerate(lens):
        k, v = kvs[b]
        for t in sorted({0, L // 2, L - 1}) if L else []:
            pg = int(bt[b, t // page])
            tt = t % page
            for h in (0, Hkv - 1):
                for d in (0, 31, 32, 63, 64, 127):
                    assert flat_k[pg, h, ((d // w) * page + tt) * w + d % w] == k[t, h, d]
                    assert flat_v[pg, h, ((tt // w) * D + d) * w + tt % w] == v[t, h, d]
        k2, v2 = unpack_request(kc, vc, bt, b, L)
        assert torch.equal(k2, k) and torch.equal(v2, v)
