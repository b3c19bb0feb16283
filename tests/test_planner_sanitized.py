"""The host planners (csrc/plan.cpp) built with g++ under the address and undefined-behaviour
sanitizers and run on random and edge-case batches: every map equals the oracle's word for word,
a buffer one word short gets the capacity status with no write past its end, and the sanitizers
report nothing.  CPU only."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.plan import ref_plan, ref_plan_lpt, ref_plan_prefill, ref_plan_static, ref_plan_weighted

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
I32_MAX = 2**31 - 1


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("planner") / "planner_sanitized")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "load_balanced_split_attn_amd", "csrc", "plan.cpp"),
           os.path.join(ROOT, "tests", "planner_sanitized.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "asan" in (res.stderr + res.stdout).lower():
        pytest.skip("sanitizer runtime not available")
    assert res.returncode == 0, res.stderr
    return out


def _cases():
    rng = np.random.default_rng(2024)
    cases = []
    # hand-picked edges: empty batch, one worker, more workers than tiles, tile 1, empty requests,
    # lengths at the int32 limit with tiles large enough to keep the tile count small
    edges = [
        (0, [], 4, 512), (0, [1024, 5120, 2048], 4, 512), (0, [0, 0, 0], 3, 64), (0, [1], 1, 1),
        (0, [7, 0, 9], 50, 1), (0, [I32_MAX, 5], 3, 2**28), (0, [I32_MAX] * 3, 7, 2**27),
        (1, [1024, 5120, 2048], 2, 512), (1, [0, 3, 0], 5, 2), (1, [I32_MAX, 1], 9, 2**28),
        (3, [1024, 5120, 2048], 4, 512), (3, [I32_MAX, 17, 0], 4, 2**28), (3, [], 2, 8),
        (4, [1024, 5120, 2048], 4, 512), (4, [I32_MAX, I32_MAX, 3], 5, 2**28), (4, [0, 0], 1, 16),
    ]
    for kind, lens, p1, tile in edges:
        extra = 256 if kind == 4 else 0
        cases.append((kind, lens, None, p1, tile, extra, 0))
    cases.append((2, [0, 5, 7], [0, 9, 30], 3, 4, 8, 1))            # prefill: empty chunk, q = kv
    cases.append((2, [3000], [I32_MAX], 2, 256, 2**26, 1))           # prefill at the int32 limit
    cases.append((2, [5, 1], [5, 40], 4, 2, 3, 0))                   # non-causal
    for _ in range(160):
        kind = int(rng.integers(0, 5))
        B = int(rng.integers(0, 30))
        big = rng.random() < 0.2
        hi = 200000 if big else 5000
        lens = [int(x) for x in rng.integers(0, hi, size=B)]
        lens = [0 if rng.random() < 0.15 else x for x in lens]
        tile = int(rng.choice([1, 7, 64, 512, 4096])) if not big else int(rng.choice([512, 4096]))
        p1 = int(rng.integers(1, 300))
        if kind == 2:
            q = [int(rng.integers(0, min(L, 600) + 1)) for L in lens]
            cases.append((2, q, lens, p1, int(rng.choice([1, 4, 128, 256])), tile, int(rng.integers(0, 2))))
        else:
            cases.append((kind, lens, None, p1, tile, int(rng.choice([0, 64, 4096])) if kind == 4 else 0, 0))
    return cases


def _oracle(kind, a, b, p1, p2, p3, p4):
    if kind == 0:
        return ref_plan(a, p1, p2)
    if kind == 1:
        return ref_plan_static(a, p1, p2)
    if kind == 2:
        return ref_plan_prefill(a, b, p1, p2, p3, bool(p4))
    if kind == 3:
        return ref_plan_lpt(a, p1, p2)
    return ref_plan_weighted(a, p1, p2, p3)


def test_planners_under_sanitizers(driver):
    lines, expected = [], []
    for kind, a, b, p1, p2, p3, p4 in _cases():
        if kind == 2:
            q_tile, kv_tile, causal = p2, p3, p4
            fields = [2, len(a), p1, q_tile, kv_tile, causal]
            ref = _oracle(2, a, b, p1, q_tile, kv_tile, causal)
            arrays = a + b
        else:
            fields = [kind, len(a), p1, p2, p3, 0]
            ref = _oracle(kind, a, None, p1, p2, p3, 0)
            arrays = a
        for short in (0, 1):
            lines.append(" ".join(str(x) for x in fields + [short] + arrays))
            expected.append((short, np.asarray(ref, dtype=np.int64), fields))
    res = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                              "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert res.returncode == 0, res.stderr[-3000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-3000:]
    out = res.stdout.strip().split("\n")
    assert len(out) == len(expected)
    for line, (short, ref, fields) in zip(out, expected):
        vals = [int(x) for x in line.split()]
        status, words = vals[0], vals[1]
        if short:
            assert status == -2, f"{fields}: one word short gave status {status}"
        else:
            assert status == 0, f"{fields}: status {status}"
            assert words == ref.size and np.array_equal(np.asarray(vals[2:], dtype=np.int64), ref), fields
