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

A pass of SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and SQ_INSTS_VALU_MFMA_MOPS_BF16 gives the
matrix cores' utilisation and the clock they ran at, per kernel:

    python -m rankmixer_block_forward_amd.counters --mfma C.csv --agents A.csv
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
    (re.compile(r"gemm_bf16_mfma(_n384)?<0[,>]"), "gemm1_gelu"),
    (re.compile(r"gemm_bf16_mfma(_n384)?<1[,>]"), "gemm2_residual"),
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


def gpu_agent(agent_csv):
    """(SIMD count, XCC count) of the first GPU agent in a rocprofv3 agent-info file."""
    with open(agent_csv, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Agent_Type") == "GPU":
                return int(row["Simd_Count"]), int(row["Num_Xcc"])
    raise SystemExit("no GPU agent in " + agent_csv)


def mfma_utilisation(counter_csv, agent_csv):
    """Matrix-core utilisation per kernel class from one counter pass of
    SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and SQ_INSTS_VALU_MFMA_MOPS_BF16.

    Per dispatch: the GPU clock in GHz is GRBM_GUI_ACTIVE (summed over the XCCs) / XCCs / the
    dispatch's duration in ns; utilisation is the MFMA busy cycles (summed over the SIMDs)
    / (SIMDs x GRBM_GUI_ACTIVE / XCCs), i.e. the fraction of the kernel's cycles in which an
    average SIMD's matrix core was busy; FLOPs are 512 x the MOPS counter.  Means over the
    dispatches of each class."""
    simds, xcc = gpu_agent(agent_csv)
    disp = defaultdict(dict)
    with open(counter_csv, newline="") as f:
        for row in csv.DictReader(f):
            k = classify(row.get("Kernel_Name", ""))
            if k is None:
                continue
            d = disp[(k, row["Dispatch_Id"])]
            d[row["Counter_Name"]] = float(row["Counter_Value"])
            d["ns"] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
    out = defaultdict(lambda: defaultdict(list))
    for (k, _), d in disp.items():
        cycles = d["GRBM_GUI_ACTIVE"] / xcc
        out[k]["ms"].append(d["ns"] / 1e6)
        out[k]["clock_ghz"].append(cycles / d["ns"])
        out[k]["mfma_busy"].append(d["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cycles))
        out[k]["tflops"].append(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / d["ns"] / 1e3)
    return {k: dict({n: sum(v) / len(v) for n, v in c.items()}, dispatches=len(c["ms"]))
            for k, c in out.items()}


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--fetch")
    p.add_argument("--write")
    p.add_argument("--workload")
    p.add_argument("--copy-bytes", type=int)
    p.add_argument("--out")
    p.add_argument("--mfma", help="counter file of an MFMA utilisation pass: print the table instead")
    p.add_argument("--agents", help="the agent-info file of the same pass (with --mfma)")
    a = p.parse_args()
    if a.mfma:
        if not a.agents:
            p.error("--mfma needs --agents")
        print("| kernel | dispatches | ms (instrumented) | clock (GHz) | MFMA busy | TFLOP/s |")
        print("|---|---|---|---|---|---|")
        for k, e in sorted(mfma_utilisation(a.mfma, a.agents).items()):
            print(f"| {k} | {e['dispatches']} | {e['ms']:.4f} | {e['clock_ghz']:.3f} | "
                  f"{100 * e['mfma_busy']:.1f}% | {e['tflops']:.1f} |")
        return
    if not (a.fetch and a.write and a.workload and a.copy_bytes and a.out):
        p.error("the traffic record needs --fetch, --write, --workload, --copy-bytes and --out")
    rec = build_record(a.fetch, a.write, a.workload, a.copy_bytes)
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
