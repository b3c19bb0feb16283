"""The measurement probes do the work their rates are computed from.

* attn_probe_stream_read and attn_probe_stream_read_rated read every 16-byte element of their buffer
  exactly once: the XOR of all per-thread digests equals the XOR of all 32-bit words of the buffer
  (an element read twice or skipped would cancel or drop its bits), for sizes with and without a
  ragged tail, and (rated) for uneven per-XCD shares, zero shares and all of it on one XCD.
* attn_probe_mfma_rate performs all blocks * 4 * iters * 8 products of 16 x 16 x 32: each thread's
  digest equals the sum, over its eight accumulators, of the entries of A.B that the matrix core
  leaves in that lane (A and B rebuilt on the host from the probe's hash, in fp64), times `iters` —
  so a compiler that dropped or merged rounds would fail — and repeated launches agree bit for bit.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import load_balanced_split_attn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


@pytest.mark.parametrize("nbytes,blocks", [(16 * 64 * 8 * 37, 3), (16 * 1000003, 64), (1 << 24, 1024)])
def test_stream_read_touches_every_element_once(lb, nbytes, blocks):
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    buf = host.cuda()
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    note(f"stream probe {nbytes} B over {blocks} blocks")
    lb.attn_probe_stream_read(buf, blocks, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("nbytes,blocks,rates", [
    (16 * 1000003, 64, [65536, 61000, 65536, 60000, 64000, 62000, 65000, 61500]),
    (1 << 24, 1024, [1, 0, 3, 0, 1, 1, 7, 2]),
    (16 * 4097, 8, [0, 0, 0, 5, 0, 0, 0, 0]),
])
def test_rated_stream_read_touches_every_element_once(lb, nbytes, blocks, rates):
    g = torch.Generator().manual_seed(nbytes + blocks)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    buf = host.cuda()
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    note(f"rated stream probe {nbytes} B over {blocks} blocks, rates {rates}")
    lb.attn_probe_stream_read_rated(buf, blocks, rates, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


def _hash(x):
    x = x.astype(np.uint32)
    x ^= x >> np.uint32(16)
    x *= np.uint32(0x7FEB352D)
    x ^= x >> np.uint32(15)
    x *= np.uint32(0x846CA68B)
    x ^= x >> np.uint32(16)
    return x


def _bf16_operands(t, offset):
    """The probe's register operand set for threads t: eight bf16 values per thread, as fp64."""
    words = np.stack([_hash(t * 32 + offset + e) for e in range(4)], axis=-1)    # [threads, 4]
    words = (words & np.uint32(0x807F807F)) | np.uint32(0x3F003F00)
    halves = np.stack([words & np.uint32(0xFFFF), words >> np.uint32(16)], axis=-1).reshape(len(t), 8)
    return (halves.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _expected_digests(blocks, iters):
    """Per-thread digest of the probe: for each wave, A (16 x 32) has row l % 16 and columns
    8 (l // 16) .. + 7 from lane l, B (32 x 16) column l % 16 and the same rows; the lane keeps
    column l % 16, rows 4 (l // 16) .. + 3 of A.B."""
    t = np.arange(blocks * 256, dtype=np.uint32)
    a = [_bf16_operands(t, 8 * k) for k in range(4)]
    b = [_bf16_operands(t, 8 * k + 4) for k in range(4)]
    lane = np.arange(64)
    out = np.zeros(blocks * 256)
    for w in range(blocks * 4):
        sl = slice(64 * w, 64 * w + 64)
        total = np.zeros(64)
        for j in range(8):
            A = np.zeros((16, 32))
            B = np.zeros((32, 16))
            for l in range(64):
                A[l % 16, 8 * (l // 16):8 * (l // 16) + 8] = a[j & 3][sl][l]
                B[8 * (l // 16):8 * (l // 16) + 8, l % 16] = b[(j >> 1) & 3][sl][l]
            D = A @ B
            total += np.array([D[4 * (l // 16):4 * (l // 16) + 4, l % 16].sum() for l in lane])
        out[sl] = total * iters
    return out


@pytest.mark.parametrize("iters", [1, 3, 257])
def test_mfma_probe_does_every_product(lb, iters):
    blocks = 2
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    note(f"mfma probe iters={iters} blocks={blocks}")
    flops = lb.attn_probe_mfma_rate(iters, blocks, sink)
    assert flops == blocks * 4 * iters * 8 * 16384
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.float32).astype(np.float64)
    want = _expected_digests(blocks, iters)
    scale = np.abs(want).max()
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) <= 1e-5 * scale * max(1, iters // 16), (got[:4], want[:4])
    again = torch.zeros_like(sink)
    lb.attn_probe_mfma_rate(iters, blocks, again)
    torch.cuda.synchronize()
    assert torch.equal(sink, again)
