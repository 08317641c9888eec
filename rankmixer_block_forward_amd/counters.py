"""HBM traffic per kernel launch from rocprofv3 counter runs.

Two counter passes of the same bench command (rocprofv3 --pmc FETCH_SIZE, then
--pmc WRITE_SIZE, both with --output-format csv) give per-dispatch KiB read from and
written to HBM through the L2.  The bench's --calibrate-copy dispatches of the token-mixing
kernel move a known number of bytes each way; what the counters read for them gives the
scale factor from counter KiB to bytes, applied to every other kernel.  The record is
keyed by the hash of the sources the GEMM kernels are compiled from, so the bench reports
it only while they are unchanged.

    python -m rankmixer_block_forward_amd.counters --fetch F.csv --write W.csv \\
        --workload "rankmixer-1b B=2048" --copy-bytes N --out profiles/traffic_counters.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
# Every source the grouped-GEMM kernels are compiled from: a record taken on other sources
# no longer describes the kernels.
GEMM_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("rmx_gemm.hip", "rmx_device.h", "rmx_internal.h")]

# kernel-name patterns -> the names the library's profiling uses
KERNELS = [
    (re.compile(r"gemm_bf16_mfma<0[,>]"), "gemm1_gelu"),
    (re.compile(r"gemm_bf16_mfma<1[,>]"), "gemm2_residual"),
    (re.compile(r"gemm_bf16_moe<2>"), "moe_ffn1"),
    (re.compile(r"gemm_bf16_moe<3>"), "moe_ffn2"),
    (re.compile(r"token_mix_kernel"), "copy"),
]


def classify(name):
    for pat, k in KERNELS:
        if pat.search(name):
            return k
    return None


def per_dispatch_kib(path, counter):
    """Mean counter value (KiB) per dispatch, by kernel class."""
    vals = defaultdict(list)
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            k = classify(row.get("Kernel_Name", ""))
            if k is not None:
                vals[k].append(float(row["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def gemm_hash():
    """First 16 hex digits of the SHA-256 of the GEMM kernels' sources, concatenated in the
    order of GEMM_SOURCES."""
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build_record(fetch_csv, write_csv, workload, copy_bytes):
    fetch = per_dispatch_kib(fetch_csv, "FETCH_SIZE")
    write = per_dispatch_kib(write_csv, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("no calibration copy dispatches in the counter files")
    f_scale = copy_bytes / (fetch["copy"][0] * 1024.0)
    w_scale = copy_bytes / (write["copy"][0] * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        if k == "copy":
            continue
        fb = fetch[k][0] * 1024.0 * f_scale
        wb = write[k][0] * 1024.0 * w_scale
        kernels[k] = {"workload": workload, "bytes_per_launch": round(fb + wb),
                      "fetch_bytes": round(fb), "write_bytes": round(wb),
                      "dispatches": [fetch[k][1], write[k][1]]}
    return {"gemm_source_sha256_16": gemm_hash(),
            "calibration": {"copy_bytes_each_way": copy_bytes,
                            "fetch_kib_read": round(fetch["copy"][0], 1),
                            "write_kib_read": round(write["copy"][0], 1),
                            "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5)},
            "kernels": kernels}


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--copy-bytes", type=int, required=True)
    p.add_argument("--out", required=True)
    a = p.parse_args()
    rec = build_record(a.fetch, a.write, a.workload, a.copy_bytes)
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
