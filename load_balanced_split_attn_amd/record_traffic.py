"""Record the HBM traffic of the split-KV kernels from two rocprofv3 counter runs.

    python -m load_balanced_split_attn_amd.record_traffic FETCH_DIR WRITE_DIR [decode|prefill]

FETCH_DIR and WRITE_DIR hold the ``*_counter_collection.csv`` of a ``--pmc FETCH_SIZE`` run and a
``--pmc WRITE_SIZE`` run of ``bench.py --calibration-copy``: on the mixed decode batch (decode, the
default; commands in ``profiles/splitkv_decode_mixed_hbm_traffic.md``) or on the chunked-prefill
batch with 128-row units and the default checked P.V (prefill; commands in
``profiles/splitkv_prefill_chunked_kernel_trace.md``).  Each counter is scaled by what it reads for
the 1 GiB calibration copy (the largest ``__amd_rocclr_copyBuffer`` dispatch of the run), the mean
over the kernel's dispatches becomes its bytes per launch, and the family's entries in
``measured_traffic.json`` are rewritten with those bytes and the digest of the kernel source they
were taken on (the other family's entries are kept); ``bench.py`` reports them as
``roofline.traffic`` only while that source is unchanged.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(PKG, "measured_traffic.json")
GIB = 1 << 30
# per kernel family: the sources its digest covers, the dispatch names (key -> kernel name), the
# workload key and the profile that documents the runs
FAMILIES = {
    "decode": {
        "sources": ("common.h", "splitkv_decode.hip"),
        "kernels": {
            "splitkv_decode_kernel": "splitkv_decode_kernel<lbsa::KvBf16, 1, 1, false>",
            "splitkv_decode_kernel_fp8": "splitkv_decode_kernel<lbsa::KvFp8, 1, 1, false>",
        },
        "workload": "mixed",
        "profile": "profiles/splitkv_decode_mixed_hbm_traffic.md",
    },
    "prefill": {
        "sources": ("common.h", "splitkv_prefill.hip"),
        # the default (checked) P.V mode with two query heads per workgroup: 128-row units
        "kernels": {"splitkv_prefill_kernel": "splitkv_prefill_kernel<1, 8, 2>"},
        "workload": "chunked_q128_checked",
        "profile": "profiles/splitkv_prefill_chunked_kernel_trace.md",
    },
}
KERNELS = FAMILIES["decode"]["kernels"]


def kernel_source_digest(family: str = "decode") -> str:
    """First 16 hex digits of the SHA-256 of a kernel family's sources (decode: common.h and
    splitkv_decode.hip; prefill: common.h and splitkv_prefill.hip)."""
    h = hashlib.sha256()
    for name in FAMILIES[family]["sources"]:
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_counter(directory: str, counter: str) -> list[tuple[str, int, float]]:
    """(kernel name, dispatch id, value in KiB summed over the counter's rows) per dispatch."""
    files = glob.glob(os.path.join(directory, "*_counter_collection.csv"))
    if not files:
        raise FileNotFoundError(f"no *_counter_collection.csv under {directory}")
    acc: dict[tuple[str, int], float] = defaultdict(float)
    for path in files:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    acc[(row["Kernel_Name"], int(row["Dispatch_Id"]))] += float(row["Counter_Value"])
    return [(k, d, v) for (k, d), v in sorted(acc.items(), key=lambda kv: kv[0][1])]


def calibration_factor(rows: list[tuple[str, int, float]]) -> float:
    copies = [v for k, _, v in rows if "copyBuffer" in k]
    if not copies:
        raise ValueError("no calibration copy in the run (bench.py --calibration-copy)")
    return GIB / (max(copies) * 1024.0)


def kernel_mean(rows: list[tuple[str, int, float]], name: str) -> float:
    vals = [v for k, _, v in rows if name in k]
    if not vals:
        raise ValueError(f"no dispatch of {name} in the run")
    return sum(vals) / len(vals)


def record(fetch_dir: str, write_dir: str, family: str = "decode", json_path: str = TRAFFIC_JSON) -> dict:
    fam = FAMILIES[family]
    workload = fam["workload"]
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")
    f_fac, w_fac = calibration_factor(fetch), calibration_factor(write)
    with open(json_path) as f:
        old = json.load(f)
    digest = kernel_source_digest(family)
    out = dict(old)
    for key, name in fam["kernels"].items():
        f_kib, w_kib = kernel_mean(fetch, name), kernel_mean(write, name)
        fetch_b, write_b = f_kib * 1024.0 * f_fac, w_kib * 1024.0 * w_fac
        entry = {
            "bytes_per_launch": int(round(fetch_b + write_b)),
            "fetch_bytes": int(round(fetch_b)),
            "write_bytes": int(round(write_b)),
            "fetch_kib_mean": round(f_kib, 2),
            "write_kib_mean": round(w_kib, 2),
            "fetch_factor": round(f_fac, 5),
            "write_factor": round(w_fac, 5),
            # the workload's algorithmic bytes do not depend on the kernel build (None where none
            # was recorded: the prefill kernel's bound is its matrix work)
            "algorithmic_bytes": old.get(key, {}).get(workload, {}).get("algorithmic_bytes"),
            "source_digest": digest,
            "profile": fam["profile"],
        }
        out[key] = {workload: entry}
    with open(json_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


if __name__ == "__main__":
    if len(sys.argv) not in (3, 4) or (len(sys.argv) == 4 and sys.argv[3] not in FAMILIES):
        sys.exit(__doc__)
    fam = sys.argv[3] if len(sys.argv) == 4 else "decode"
    out = record(sys.argv[1], sys.argv[2], fam)
    for key in FAMILIES[fam]["kernels"]:
        e = out[key][FAMILIES[fam]["workload"]]
        ratio = (f", {e['bytes_per_launch'] / e['algorithmic_bytes']:.4f}x algorithmic"
                 if e["algorithmic_bytes"] else "")
        print(f"{key}: {e['bytes_per_launch']} B per launch{ratio} (fetch {e['fetch_kib_mean']} KiB x "
              f"{e['fetch_factor']}, write {e['write_kib_mean']} KiB)")
