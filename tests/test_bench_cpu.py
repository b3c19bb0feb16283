"""CPU checks of the measurement arithmetic in bench.py: algorithmic bytes per step (against totals
worked out by hand from the workload definitions), prefill flops (against a brute-force count of
visible (row, key) pairs), the per-CU busy union (against synthetic timestamp records), and that an
optional comparison section records its error instead of ending the run."""

import numpy as np
import pytest
import torch

import bench
import workloads as WL


@pytest.mark.parametrize("name,expected", [
    # KV 4096 B per token (8 heads x 128 dims x 2 B x K and V) + Q 16 KiB and fp32 out 32 KiB per
    # request + 4 B per 64-token page + 4 B per length
    ("tiny", 8192 * 4096 + 3 * 16384 + 3 * 32768 + 128 * 4 + 3 * 4),                 # 33,702,412
    ("uniform", 64 * 8192 * 4096 + 64 * 16384 + 64 * 32768 + 64 * 128 * 4 + 64 * 4),  # 2,150,662,400
    ("mixed", 1744896 * 4096 + 40 * 16384 + 40 * 32768 + 27264 * 4 + 40 * 4),         # 7,149,169,312
])
def test_step_bytes(name, expected):
    nb = bench.algorithmic_bytes(WL.BY_NAME[name](), 64)
    assert nb["step"] == expected
    assert nb["splitkv"] == expected - nb["out"]
    assert nb["out"] == WL.BY_NAME[name]().batch * 64 * 128 * 4


def test_step_bytes_fixed_values():
    assert bench.algorithmic_bytes(WL.tiny(), 64)["step"] == 33_702_412
    assert bench.algorithmic_bytes(WL.uniform(), 64)["step"] == 2_150_662_400
    assert bench.algorithmic_bytes(WL.mixed(), 64)["step"] == 7_149_169_312
    assert bench.algorithmic_bytes(WL.mixed(), 64)["splitkv"] == 7_147_858_592


def test_step_bytes_fp8_and_head_share():
    wl = WL.mixed()
    nb8 = bench.algorithmic_bytes(wl, 64, kv_elem=1)
    assert nb8["kv"] == 1744896 * 2048 + 2 * 8 * 4          # codes + one fp32 scale per head for K and V
    share = WL.mixed_tp8()
    nbs = bench.algorithmic_bytes(share, 64)
    assert nbs["kv"] == 1744896 * 512                       # one KV head
    assert nbs["q"] == 40 * 8 * 128 * 2 and nbs["out"] == 40 * 8 * 128 * 4


def test_prefill_flops_brute_force():
    class W:
        head_dim, hq = 128, 64
        q_lens = [2, 5, 1, 7]
        kv_lens = [5, 5, 9, 7]
    pairs = 0
    for ql, kl in zip(W.q_lens, W.kv_lens):
        for j in range(ql):
            pos = kl - ql + j
            pairs += sum(1 for t in range(kl) if t <= pos)
    assert bench.prefill_flops(W) == 4 * 128 * 64 * pairs


def _rec(start, end, cu, se=0, sh=0, xcc=0, wave=0, simd=0):
    hw = (se << 13) | (sh << 12) | (cu << 8) | (simd << 4) | wave
    return [start, end, hw, xcc]


def test_per_cu_busy_union():
    recs = [
        _rec(0, 10, cu=1), _rec(5, 20, cu=1, simd=2, wave=3),    # one CU, overlapping: busy 20
        _rec(30, 40, cu=1, simd=1),                                # same CU later: +10 -> 30
        _rec(0, 10, cu=2),                                         # another CU: 10
        _rec(0, 10, cu=1, xcc=3),                                  # same CU id on another XCD: 10
        _rec(2, 4, cu=1, se=1), _rec(4, 8, cu=1, se=1),            # touching intervals: 6
    ]
    r = bench.per_cu_busy(torch.tensor(recs, dtype=torch.int64))
    busy = np.array([30, 10, 10, 6], dtype=np.float64)
    assert r["cus_seen"] == 4
    assert r["workgroups"] == len(recs)
    assert r["max_over_mean"] == pytest.approx(busy.max() / busy.mean())
    assert r["tail_fraction"] == pytest.approx((busy.max() - busy.mean()) / busy.max())
    assert r["mean_busy_over_span"] == pytest.approx(busy.mean() / 40)


def test_optional_section_records_errors():
    """A comparison section that fails records its error in the line; one that works returns its
    result unchanged."""
    assert bench.optional_section("ok", lambda: {"x": 1}) == {"x": 1}

    def broken():
        raise ValueError("no timed workgroup ran on XCD 3")

    got = bench.optional_section("broken", broken)
    assert got == {"error": "ValueError: no timed workgroup ran on XCD 3"}
