"""Oracle attention pinned against brute force, closed forms, a library routine and the
combine invariant (see tests/oracle_pins.py)."""

import numpy as np
import pytest

import oracle_pins as P
from oracle.attention import (ref_attention, ref_combine, ref_decode, ref_from_map, ref_partial,
                              ref_split_partials)
from oracle.plan import ref_plan, ref_plan_prefill, ref_plan_static


def test_bruteforce_decode():
    P.pin_bruteforce_decode(ref_attention)


def test_bruteforce_prefill():
    P.pin_bruteforce_prefill(ref_attention)


def test_closed_forms():
    P.pin_closed_forms(ref_attention)


def test_gqa_head_map():
    P.pin_gqa_head_map(ref_attention)


def test_library_sdpa():
    P.pin_library_sdpa(ref_attention)


def test_combine_invariance():
    P.pin_combine_invariance(ref_attention, ref_partial, ref_combine)


def test_partial_definition():
    P.pin_partial_definition(ref_partial)


def test_empty_request_gives_zero():
    q = np.ones((1, 8, 4))
    k = np.zeros((0, 2, 4))
    out = ref_attention(q, k, k, 1.0)
    assert out.shape == (1, 8, 4) and np.all(out == 0)


def test_prefill_row_equals_decode_at_its_position():
    """A chunk row j is a decode query at position P + j over keys [0, P + j]."""
    rng = np.random.default_rng(4)
    Pfx, R = 23, 6
    q = rng.standard_normal((R, 8, 16))
    k = rng.standard_normal((Pfx + R, 2, 16))
    v = rng.standard_normal((Pfx + R, 2, 16))
    out = ref_attention(q, k, v, 0.3, causal=True)
    for j in range(R):
        dec = ref_attention(q[j:j + 1], k[:Pfx + j + 1], v[:Pfx + j + 1], 0.3, causal=True)
        assert np.allclose(out[j], dec[0], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("W", [1, 3, 4, 7, 64])
def test_map_split_equals_unsplit_decode(W):
    rng = np.random.default_rng(W)
    lens = [0, 1, 17, 130, 64, 300]
    q = rng.standard_normal((len(lens), 8, 16))
    ks = [rng.standard_normal((L, 2, 16)) for L in lens]
    vs = [rng.standard_normal((L, 2, 16)) for L in lens]
    exp = ref_decode(q, ks, vs, 0.25)
    for words in (ref_plan(lens, W, 32), ref_plan_static(lens, max(1, W // 2), 32)):
        outs = ref_from_map(words, [q[b:b + 1] for b in range(len(lens))], ks, vs, 0.25)
        got = np.stack([o[0] for o in outs])
        assert np.allclose(got, exp, rtol=1e-13, atol=1e-13)


def test_map_split_equals_unsplit_prefill():
    rng = np.random.default_rng(9)
    q_lens, kv_lens = [5, 1, 9], [40, 1, 9]
    qs = [rng.standard_normal((ql, 8, 8)) for ql in q_lens]
    ks = [rng.standard_normal((L, 2, 8)) for L in kv_lens]
    vs = [rng.standard_normal((L, 2, 8)) for L in kv_lens]
    for causal in (True, False):
        words = ref_plan_prefill(q_lens, kv_lens, 5, 4, 8, causal)
        outs = ref_from_map(words, qs, ks, vs, 0.5, causal)
        for b in range(3):
            exp = ref_attention(qs[b], ks[b], vs[b], 0.5, causal=causal)
            assert np.allclose(outs[b], exp, rtol=1e-13, atol=1e-13)
        parts = ref_split_partials(words, qs, ks, vs, 0.5, causal)
        assert len(parts) == int(words[4])
