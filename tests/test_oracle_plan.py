"""Oracle work-map builder pinned against the pages' worked example, the budget rule, a
closed-form fill, structural invariants and edge cases."""

import numpy as np
import pytest

import oracle_pins as P
from oracle.plan import (map_words, parse_map, ref_plan, ref_plan_prefill, ref_plan_static,
                         tiles_of)


def test_worked_example_pages():
    P.pin_worked_example(ref_plan, parse_map)


def test_worked_example_placement_reading():
    """Placement under the contiguous-fill reading (the figure itself is not in the text)."""
    mp = parse_map(ref_plan([1024, 5120, 2048], 4, 512))
    assert [mp.worker_segments(w).tolist() for w in range(4)] == [
        [[0, 0, 0, 1024], [1, 0, 0, 1024]],
        [[1, 0, 1024, 3072]],
        [[1, 0, 3072, 5120]],
        [[2, 0, 0, 2048]],
    ]
    assert mp.unit_ptr.tolist() == [0, 1, 4, 5]
    assert mp.units.tolist() == [[0, 0], [1, 0], [2, 0]]
    assert (mp.version, mp.B, mp.W, mp.kv_tile, mp.S, mp.T, mp.q_tile, mp.U) == (1, 3, 4, 512, 5, 16, 1, 3)


def test_fill_closed_form():
    P.pin_fill_closed_form(ref_plan, parse_map)


def test_budget_rule():
    P.pin_budget_rule(ref_plan, parse_map)


def _check_invariants(words, extents, tile):
    mp = parse_map(words)
    assert mp.version == 1
    assert len(words) == map_words(mp.U, mp.W, mp.S)
    assert np.all(np.diff(mp.worker_ptr) >= 0) and mp.worker_ptr[0] == 0 and mp.worker_ptr[-1] == mp.S
    assert np.all(np.diff(mp.unit_ptr) >= 0) and mp.unit_ptr[0] == 0 and mp.unit_ptr[-1] == mp.S
    T = sum(tiles_of(e, tile) for e in extents)
    assert mp.T == T
    seen = []
    for u in range(mp.U):
        b, i = mp.units[u]
        segs = mp.unit_segments(u)
        cursor = 0
        for sb, si, a, e in segs:
            assert (sb, si) == (b, i)
            assert a == cursor and a % tile == 0 and a < e <= extents[u]
            assert e == extents[u] or e % tile == 0
            cursor = e
            seen += [(u, t) for t in range(a // tile, -(-e // tile))]
        assert cursor == extents[u]
    assert len(seen) == T == len(set(seen))
    if T:
        assert mp.S <= min(T, mp.W + mp.U - 1)
    # worker lists concatenated are the stream in order
    order = []
    for w in range(mp.W):
        for sb, si, a, e in mp.worker_segments(w):
            order.append((sb, si, a))
    assert order == sorted(order)


def test_invariants_random_decode():
    rng = np.random.default_rng(1)
    for trial in range(10000):
        B = int(rng.integers(0, 12))
        tile = int(rng.choice([1, 2, 7, 64, 512]))
        lens = [int(x) for x in rng.integers(0, 8 * tile + 3, size=B)]
        W = int(rng.integers(1, 50))
        _check_invariants(ref_plan(lens, W, tile), lens, tile)


def test_invariants_random_prefill():
    rng = np.random.default_rng(2)
    for trial in range(2000):
        B = int(rng.integers(0, 5))
        q_lens = [int(x) for x in rng.integers(0, 40, size=B)]
        kv_lens = [q + int(rng.integers(0, 100)) for q in q_lens]
        q_tile = int(rng.choice([1, 4, 16]))
        kv_tile = int(rng.choice([3, 8, 32]))
        causal = bool(rng.integers(0, 2))
        W = int(rng.integers(1, 30))
        words = ref_plan_prefill(q_lens, kv_lens, W, q_tile, kv_tile, causal)
        extents = []
        for ql, kl in zip(q_lens, kv_lens):
            for i in range(-(-ql // q_tile)):
                extents.append(kl - ql + min(ql, (i + 1) * q_tile) if causal else kl)
        _check_invariants(words, extents, kv_tile)


def test_static_chunks():
    rng = np.random.default_rng(3)
    for trial in range(2000):
        lens = [int(x) for x in rng.integers(0, 20 * 64, size=int(rng.integers(0, 8)))]
        S = int(rng.integers(1, 9))
        words = ref_plan_static(lens, S, 64)
        _check_invariants(words, lens, 64)
        mp = parse_map(words)
        assert mp.W == mp.S == sum(min(S, tiles_of(L, 64)) for L in lens)
        for u, L in enumerate(lens):
            sizes = [-(-(int(e) - int(a)) // 64) for _, _, a, e in mp.unit_segments(u)]
            assert len(sizes) == min(S, tiles_of(L, 64))
            if sizes:
                assert max(sizes) - min(sizes) <= 1 and sizes == sorted(sizes, reverse=True)


def test_static_example():
    mp = parse_map(ref_plan_static([1024, 5120, 2048], 2, 512))
    assert mp.segs.tolist() == [[0, 0, 0, 512], [0, 0, 512, 1024], [1, 0, 0, 2560], [1, 0, 2560, 5120],
                                [2, 0, 0, 1024], [2, 0, 1024, 2048]]


def test_edge_cases():
    mp = parse_map(ref_plan([], 4, 512))
    assert (mp.B, mp.S, mp.T, mp.U) == (0, 0, 0, 0) and mp.worker_ptr.tolist() == [0] * 5
    mp = parse_map(ref_plan([0, 0], 3, 512))
    assert mp.S == 0 and mp.unit_ptr.tolist() == [0, 0, 0]
    mp = parse_map(ref_plan([100], 8, 512))          # more workers than tiles
    assert mp.worker_ptr.tolist() == [0, 1, 1, 1, 1, 1, 1, 1, 1] and mp.segs.tolist() == [[0, 0, 0, 100]]
    mp = parse_map(ref_plan([513], 1, 512))           # ragged tail, one worker
    assert mp.segs.tolist() == [[0, 0, 0, 513]] and mp.T == 2
    with pytest.raises(ValueError):
        ref_plan([-1], 2, 512)
    with pytest.raises(ValueError):
        ref_plan([5], 0, 512)
    with pytest.raises(ValueError):
        ref_plan([5], 2, 0)
    with pytest.raises(ValueError):
        ref_plan_prefill([5], [4], 2, 4, 8, True)      # chunk longer than the context


def test_prefill_extents():
    # q_len 300 after a 700-token prefix, q_tile 128: rows 0-127 see up to 828 keys, etc.
    mp = parse_map(ref_plan_prefill([300, 128], [1000, 128], 3, 128, 512, True))
    assert mp.units.tolist() == [[0, 0], [0, 1], [0, 2], [1, 0]]
    ends = {}
    for b, i, a, e in mp.segs.tolist():
        ends[(b, i)] = max(ends.get((b, i), 0), e)
    assert ends == {(0, 0): 828, (0, 1): 956, (0, 2): 1000, (1, 0): 128}


def test_lpt_coverage_and_balance():
    from oracle.plan import parse_map, ref_plan_lpt
    P.pin_lpt_coverage_and_balance(ref_plan_lpt, parse_map)


def test_lpt_equal_sizes_round_robin():
    from oracle.plan import parse_map, ref_plan_lpt
    P.pin_lpt_equal_sizes_round_robin(ref_plan_lpt, parse_map)


def test_lpt_hand_example():
    from oracle.plan import parse_map, ref_plan_lpt
    P.pin_lpt_hand_example(ref_plan_lpt, parse_map)


def test_weighted_contiguous_and_balanced():
    from oracle.plan import parse_map, ref_plan_weighted
    P.pin_weighted_contiguous_and_balanced(ref_plan_weighted, parse_map)


def test_weighted_worked_example():
    from oracle.plan import parse_map, ref_plan_weighted
    P.pin_weighted_worked_example(ref_plan_weighted, parse_map)


def test_weighted_hand_examples():
    from oracle.plan import parse_map, ref_plan_weighted
    P.pin_weighted_hand_examples(ref_plan_weighted, parse_map)


def test_weighted_rejects_negative_split_cost():
    import pytest
    from oracle.plan import ref_plan_weighted
    with pytest.raises(ValueError):
        ref_plan_weighted([100], 2, 64, -1)


def test_rated_equal_rates_are_weighted():
    from oracle.plan import ref_plan_rated, ref_plan_weighted
    P.pin_rated_equal_rates_are_weighted(ref_plan_rated, ref_plan_weighted)


def test_rated_contiguous_and_proportional():
    from oracle.plan import parse_map, ref_plan_rated
    P.pin_rated_contiguous_and_proportional(ref_plan_rated, parse_map)


def test_rated_hand_examples():
    from oracle.plan import parse_map, ref_plan_rated
    P.pin_rated_hand_examples(ref_plan_rated, parse_map)


def test_rated_rejects_bad_rates():
    from oracle.plan import RATE_MAX, ref_plan_rated
    for rates in ([1, 2], [0, 0, 0], [1, -1, 1], [1, RATE_MAX + 1, 1]):
        with pytest.raises(ValueError):
            ref_plan_rated([100, 200], 3, 512, 0, rates)
    with pytest.raises(ValueError):
        ref_plan_rated([100, 200], 3, 512, -1, [1, 1, 1])

