"""The traffic recorder on synthetic rocprofv3 counter files: calibration by the largest copy,
mean over the kernel's dispatches, rows of one dispatch summed, the workload's algorithmic bytes
kept, the decode source's digest stamped; the prefill family beside it."""

import csv
import json
import os

import pytest

from load_balanced_split_attn_amd import record_traffic as RT

BF16 = "void lbsa::splitkv_decode_kernel<lbsa::KvBf16, 1, 1, false>(lbsa::DecodeParams)"
FP8 = "void lbsa::splitkv_decode_kernel<lbsa::KvFp8, 1, 1, false>(lbsa::DecodeParams)"
COPY = "__amd_rocclr_copyBuffer"


def _write(directory, counter, rows):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, k, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_record(tmp_path):
    # fetch: the 1 GiB copy reads half its bytes (factor 2); a small copy must not be the calibration
    _write(tmp_path / "f", "FETCH_SIZE", [(1, COPY, 512 * 1024), (2, COPY, 1000), (3, BF16, 100.0), (3, BF16, 50.0),
                                          (4, BF16, 170.0), (5, FP8, 40.0), (6, FP8, 60.0)])
    _write(tmp_path / "w", "WRITE_SIZE", [(1, COPY, 1024 * 1024), (2, COPY, 2000), (3, BF16, 4.0), (4, BF16, 6.0),
                                          (5, FP8, 2.0), (6, FP8, 2.0)])
    js = tmp_path / "t.json"
    js.write_text(json.dumps({"splitkv_decode_kernel": {"mixed": {"algorithmic_bytes": 111}},
                              "splitkv_decode_kernel_fp8": {"mixed": {"algorithmic_bytes": 222}}}))
    out = RT.record(str(tmp_path / "f"), str(tmp_path / "w"), json_path=str(js))
    b = out["splitkv_decode_kernel"]["mixed"]
    assert b["fetch_factor"] == 2.0 and b["write_factor"] == 1.0
    assert b["fetch_kib_mean"] == 160.0 and b["write_kib_mean"] == 5.0     # (150 + 170) / 2, (4 + 6) / 2
    assert b["fetch_bytes"] == 160 * 1024 * 2 and b["write_bytes"] == 5 * 1024
    assert b["bytes_per_launch"] == b["fetch_bytes"] + b["write_bytes"]
    assert b["algorithmic_bytes"] == 111
    assert b["source_digest"] == RT.kernel_source_digest()
    f = out["splitkv_decode_kernel_fp8"]["mixed"]
    assert f["fetch_bytes"] == 50 * 1024 * 2 and f["write_bytes"] == 2 * 1024 and f["algorithmic_bytes"] == 222
    assert json.loads(js.read_text()) == out


def test_missing_pieces(tmp_path):
    _write(tmp_path / "f", "FETCH_SIZE", [(1, BF16, 1.0)])
    _write(tmp_path / "w", "WRITE_SIZE", [(1, COPY, 1024 * 1024), (2, BF16, 1.0)])
    js = tmp_path / "t.json"
    js.write_text("{}")
    with pytest.raises(ValueError, match="calibration"):
        RT.record(str(tmp_path / "f"), str(tmp_path / "w"), json_path=str(js))
    with pytest.raises(FileNotFoundError):
        RT.read_counter(str(tmp_path / "none"), "FETCH_SIZE")


def test_record_prefill_keeps_decode(tmp_path):
    # the prefill family rewrites only its own entry, stamped with the prefill sources' digest
    pf = "void lbsa::splitkv_prefill_kernel<1, 8, 2>(lbsa::PrefillParams)"
    other = "void lbsa::splitkv_prefill_kernel<1, 8, 1>(lbsa::PrefillParams)"
    _write(tmp_path / "f", "FETCH_SIZE", [(1, COPY, 512 * 1024), (2, pf, 300.0), (3, pf, 100.0), (4, other, 7.0)])
    _write(tmp_path / "w", "WRITE_SIZE", [(1, COPY, 1024 * 1024), (2, pf, 8.0), (3, pf, 8.0), (4, other, 1.0)])
    js = tmp_path / "t.json"
    decode = {"splitkv_decode_kernel": {"mixed": {"algorithmic_bytes": 111, "bytes_per_launch": 5}}}
    js.write_text(json.dumps(decode))
    out = RT.record(str(tmp_path / "f"), str(tmp_path / "w"), family="prefill", json_path=str(js))
    e = out["splitkv_prefill_kernel"]["chunked_q128_checked"]
    assert e["fetch_bytes"] == 200 * 1024 * 2 and e["write_bytes"] == 8 * 1024   # the 8-wave, 2-head launches only
    assert e["algorithmic_bytes"] is None
    assert e["source_digest"] == RT.kernel_source_digest("prefill") != RT.kernel_source_digest("decode")
    assert out["splitkv_decode_kernel"] == decode["splitkv_decode_kernel"]
    assert json.loads(js.read_text()) == out
