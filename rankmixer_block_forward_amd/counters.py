"""Memory traffic per kernel launch from rocprofv3 counter runs.

The traffic record counts the requests the L2 (TCC) sends to memory, by size.  One counter
pass of a bench command with TCC_EA0_RDREQ_sum, TCC_EA0_RDREQ_32B_sum,
TCC_EA0_RDREQ_64B_sum and TCC_EA0_RDREQ_128B_sum (--output-format csv), and one with
TCC_EA0_WRREQ_sum and TCC_EA0_WRREQ_64B_sum, give per dispatch
    read bytes  = 32 n32 + 64 n64 + 128 n128
    write bytes = 64 n64w + 32 (n_w - n64w).
These are the bytes that leave the L2 towards the memory fabric (the 256 MB memory-side
cache and HBM behind it; the counters cannot tell which of the two served a request).
No scale factor enters.  The derived FETCH_SIZE counter of this part prices 128-byte reads
through TCC_BUBBLE, which reads 0 on gfx950, and so reports half of every 128-byte read.

    python -m rankmixer_block_forward_amd.counters --reads R.csv --writes W.csv \\
        --workload "rankmixer-1b B=2048" --out profiles/traffic_counters.json

FETCH_SIZE / WRITE_SIZE passes scaled by a plain streaming copy of known size (the bench's
--calibrate-copy dispatches) give the same figures for kernels whose reads are all 128-byte
requests:

    python -m rankmixer_block_forward_amd.counters --fetch F.csv --write W.csv \\
        --workload "rankmixer-1b B=2048" --copy-bytes N

The record is keyed by the hash of the sources the GEMM kernels are compiled from, so the
bench reports it only while they are unchanged.

Per-kernel durations of a kernel-trace run (rocprofv3 --kernel-trace --stats; the results
database):

    python -m rankmixer_block_forward_amd.counters --stats run_results.db

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
GEMM_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("rmx_gemm.hip", "rmx_device.h", "rmx_internal.h", "rmx_layout.h")]

# kernel-name patterns -> the names the library's profiling uses
KERNELS = [
    (re.compile(r"gemm_bf16_mfma(_n384|_n192|_m64|_w8)?<0[,>]"), "gemm1_gelu"),
    (re.compile(r"gemm_bf16_mfma(_n384|_n192|_m64|_w8)?<1[,>]"), "gemm2_residual"),
    (re.compile(r"gemm_bf16_moe(_n384)?<2>"), "moe_ffn1"),
    (re.compile(r"gemm_bf16_moe(_n384)?<3>"), "moe_ffn2"),
    (re.compile(r"rows_kernel<[^>]*, 0(, (false|true))?>"), "rows_first"),
    (re.compile(r"rows_kernel<[^>]*, 1(, (false|true))?>"), "rows_ln2_mix_ln1"),
    (re.compile(r"rows_kernel<[^>]*, 2(, (false|true))?>"), "rows_ln2_pool"),
    (re.compile(r"vectorized_elementwise_kernel<\d+, at::native::neg_kernel"), "copy"),
]


def classify(name):
    for pat, k in KERNELS:
        if pat.search(name):
            return k
    return None


def per_dispatch_kib(path, counter):
    """Mean counter value per dispatch, by kernel class: {class: (mean, dispatches)}."""
    vals = defaultdict(list)
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            k = classify(row.get("Kernel_Name", ""))
            if k is not None:
                vals[k].append(float(row["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def request_bytes(reads_csv, writes_csv):
    """Bytes read and written per dispatch, by kernel class, from the request counts by size:
    {class: {"read": bytes, "write": bytes, "dispatches": n, "read_requests": {...}}}."""
    n32 = per_dispatch_kib(reads_csv, "TCC_EA0_RDREQ_32B_sum")
    n64 = per_dispatch_kib(reads_csv, "TCC_EA0_RDREQ_64B_sum")
    n128 = per_dispatch_kib(reads_csv, "TCC_EA0_RDREQ_128B_sum")
    ntot = per_dispatch_kib(reads_csv, "TCC_EA0_RDREQ_sum")
    w_all = per_dispatch_kib(writes_csv, "TCC_EA0_WRREQ_sum")
    w64 = per_dispatch_kib(writes_csv, "TCC_EA0_WRREQ_64B_sum")
    out = {}
    for k in sorted(set(n128) & set(w_all)):
        a, b, c = n32.get(k, (0.0, 0))[0], n64.get(k, (0.0, 0))[0], n128[k][0]
        wa, wb = w_all[k][0], w64.get(k, (0.0, 0))[0]
        out[k] = {"read": 32.0 * a + 64.0 * b + 128.0 * c, "write": 64.0 * wb + 32.0 * (wa - wb),
                  "dispatches": [n128[k][1], w_all[k][1]],
                  "read_requests": {"32B": a, "64B": b, "128B": c, "all": ntot.get(k, (0.0, 0))[0]}}
    return out


def build_request_record(reads_csv, writes_csv, workload):
    """The traffic record (bytes per launch by kernel class) from the request-size passes."""
    kernels = {}
    for k, e in request_bytes(reads_csv, writes_csv).items():
        if k == "copy":
            continue
        kernels[k] = {"workload": workload, "bytes_per_launch": round(e["read"] + e["write"]),
                      "read_bytes": round(e["read"]), "write_bytes": round(e["write"]),
                      "dispatches": e["dispatches"]}
    return {"gemm_source_sha256_16": gemm_hash(),
            "method": "L2-to-memory requests by size (TCC_EA0_RDREQ_32B/64B/128B, TCC_EA0_WRREQ/_64B)",
            "kernels": kernels}


def kernel_stats(db_path):
    """Per-kernel totals of a rocprofv3 kernel-trace results database: a list of
    (kernel name, calls, total us, average us, percentage, min us, max us), longest total
    first (min and max from the per-dispatch durations, in ns in the database)."""
    import sqlite3
    con = sqlite3.connect(db_path)
    try:
        rows = con.execute("select name, total_calls, total_duration, average, percentage from top_kernels "
                           "order by total_duration desc").fetchall()
        ext = {}
        try:
            for name, lo, hi in con.execute("select name, min(duration), max(duration) from kernels group by name"):
                ext[name] = (lo / 1e3, hi / 1e3)
        except sqlite3.Error:
            pass
    finally:
        con.close()
    return [tuple(r) + ext.get(r[0], (float("nan"), float("nan"))) for r in rows]


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
    p.add_argument("--reads", help="counter file of the read-request pass")
    p.add_argument("--writes", help="counter file of the write-request pass")
    p.add_argument("--fetch")
    p.add_argument("--write")
    p.add_argument("--workload")
    p.add_argument("--copy-bytes", type=int)
    p.add_argument("--out")
    p.add_argument("--stats", help="rocprofv3 kernel-trace results database: print the kernel table instead")
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
    if a.stats:
        print("| kernel | calls | average (us) | min (us) | max (us) | total (ms) | share |")
        print("|---|---|---|---|---|---|---|")
        for name, calls, total, avg, pct, lo, hi in kernel_stats(a.stats):
            short = re.sub(r"^void |\(.*$|rmx::\(anonymous namespace\)::", "", name)
            print(f"| `{short}` | {calls} | {avg:.1f} | {lo:.1f} | {hi:.1f} | {total / 1e3:.3f} | {pct:.1f}% |")
        return
    if a.reads and a.writes and a.workload:
        rec = build_request_record(a.reads, a.writes, a.workload)
        if a.out:
            with open(a.out, "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
        print(json.dumps(rec, indent=1))
        return
    if not (a.fetch and a.write and a.workload and a.copy_bytes):
        p.error("give --reads, --writes and --workload (request counts), or --fetch, --write, --workload "
                "and --copy-bytes (scaled FETCH_SIZE / WRITE_SIZE)")
    rec = build_record(a.fetch, a.write, a.workload, a.copy_bytes)
    if a.out:
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
