"""The device-built work map (attn_plan_device): bit-exact with the oracle's map on random batches,
device-side error reporting, and a whole decode step (plan + split-KV + combine) captured in one
HIP graph and replayed with new lengths, checked against the fp64 oracle after every replay."""

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_helpers import SCALE, assert_close, decode_inputs, note
from oracle.attention import ref_attention
from oracle.plan import ref_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _device_map(lb, lens, W, tile, words=None):
    dev = torch.device("cuda")
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    cap = words if words is not None else lb.device_map_words(len(lens), W)
    m = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    lb.attn_plan_device(lens_d, W, tile, m)
    torch.cuda.synchronize()
    return m.cpu().numpy()


def test_bit_exact_random_batches(lb):
    rng = np.random.default_rng(17)
    cases = 0
    for trial in range(1200):
        B = int(rng.choice([0, 1, 2, 3, 7, 40, 333, 1500, 3000]))
        W = int(rng.choice([1, 2, 3, 5, 64, 128, 256, 1000, 2048]))
        tile = int(rng.choice([16, 64, 512, 4096]))
        # total tiles kept to a few hundred thousand so the oracle's explicit stream stays quick
        top = 300000 if B <= 40 else 4000
        kind = rng.integers(0, 4, size=B)
        lens = np.where(kind == 0, 0, np.where(kind == 1, rng.integers(1, 600, size=B),
                        np.where(kind == 2, rng.integers(0, 20000, size=B) % top, rng.integers(0, top, size=B))))
        lens = [int(x) for x in lens]
        exp = np.asarray(ref_plan(lens, W, tile), dtype=np.int32)
        got = _device_map(lb, lens, W, tile)
        assert np.array_equal(got[:exp.size], exp), f"B={B} W={W} tile={tile}"
        assert np.array_equal(lb.attn_plan(lens, W, tile), exp)
        cases += 1
    note(f"{cases} random batches bit-exact")


def test_full_size_workloads(lb):
    for name in ("tiny", "uniform", "mixed", "long_tail"):
        wl = WL.BY_NAME[name]()
        W = wl.workers or 128
        exp = np.asarray(ref_plan(wl.kv_lens, W, 512), dtype=np.int32)
        got = _device_map(lb, wl.kv_lens, W, 512)
        assert np.array_equal(got[:exp.size], exp), name


def test_device_errors(lb):
    got = _device_map(lb, [5, -1, 7], 4, 512)
    assert got[0] == -1                                  # LBSA_ERR_INVALID: negative length
    lens = [5000] * 6                                    # 60 tiles over 7 workers: S = 12 segments
    exp = ref_plan(lens, 7, 512)
    S = int(exp[4])
    fixed = 8 + 8 + 7 + 12
    got = _device_map(lb, lens, 7, 512, words=fixed + 4 * (S - 1))
    assert got[0] == -2 and got[4] == S                  # LBSA_ERR_CAPACITY with the count needed
    # a map reporting an error makes the split and combine kernels do nothing
    from load_balanced_split_attn_amd.decode import DeviceDecodeStep
    wl = WL.random_decode(30, 3, 900, min_len=1)
    q, kc, vc, bt = decode_inputs(wl)
    step = DeviceDecodeStep(wl.batch, q.device, num_workers=4)
    step.seq_lens.copy_(torch.tensor([5, -3, 9], dtype=torch.int32))
    out = torch.full(q.shape, 123.0, dtype=torch.float32, device=q.device)
    step(q, kc, vc, bt, scale=SCALE, out=out)
    torch.cuda.synchronize()
    assert int(step.map[0].item()) == -1 and bool(torch.all(out == 123.0))


def test_graph_captured_step(lb):
    from load_balanced_split_attn_amd.decode import DeviceDecodeStep
    wl = WL.random_decode(31, 6, 4000, min_len=800)
    q, kc, vc, bt = decode_inputs(wl)
    dev = q.device
    step = DeviceDecodeStep(wl.batch, dev, num_workers=48)
    out = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    step.seq_lens.copy_(torch.tensor(wl.kv_lens, dtype=torch.int32))
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
    qd = wl.q().double().numpy()
    kvs = [wl.kv(b) for b in range(wl.batch)]
    rng = np.random.default_rng(5)
    for replay in range(4):
        # new lengths (a prefix of each request's cache, some empty), set on the device, then replay
        new = [int(rng.integers(0, L + 1)) if replay else L for L in wl.kv_lens]
        if replay == 2:
            new[0] = 0
        step.seq_lens.copy_(torch.tensor(new, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(step.map.cpu().numpy()[:len(ref_plan(new, 48, 512))], ref_plan(new, 48, 512))
        got = out.cpu().numpy()
        for b, L in enumerate(new):
            k, v = kvs[b]
            ref = ref_attention(qd[b:b + 1], k[:L].double().numpy(), v[:L].double().numpy(), SCALE)[0]
            assert_close(got[b], ref, f"replay {replay} request {b} (L={L})")
        note(f"replay {replay}: lengths {new} ok")
