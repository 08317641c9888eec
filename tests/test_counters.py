"""Host logic of the HBM traffic record (rankmixer_block_forward_amd/counters.py): the
calibration scale comes from the copy dispatches and is applied per kernel."""
import csv
import json

from rankmixer_block_forward_amd import counters


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_record_scales_by_copy_calibration(tmp_path):
    g1 = "void rmx::(anonymous namespace)::gemm_bf16_mfma<0>(rmx::GemmArgs)"
    g2 = "void rmx::(anonymous namespace)::gemm_bf16_mfma_n384<1>(rmx::GemmArgs)"
    cp = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)::{lambda(float)#1}>(...)"
    other = "void at::native::vectorized_elementwise_kernel<4>(...)"
    copy_bytes = 1 << 30
    # the fetch counter reads 5/6 of the copy, the write counter all of it
    _write(tmp_path / "f.csv", [(cp, "FETCH_SIZE", copy_bytes / 1024 * 5 / 6)] * 3 +
           [(g1, "FETCH_SIZE", 1000.0), (g1, "FETCH_SIZE", 3000.0), (g2, "FETCH_SIZE", 600.0),
            (other, "FETCH_SIZE", 1e9)])
    _write(tmp_path / "w.csv", [(cp, "WRITE_SIZE", copy_bytes / 1024)] * 3 +
           [(g1, "WRITE_SIZE", 500.0), (g1, "WRITE_SIZE", 500.0), (g2, "WRITE_SIZE", 100.0)])
    rec = counters.build_record(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "w B=1", copy_bytes)
    assert abs(rec["calibration"]["fetch_scale"] - 1.2) < 1e-4
    assert abs(rec["calibration"]["write_scale"] - 1.0) < 1e-9
    k1 = rec["kernels"]["gemm1_gelu"]
    assert k1["fetch_bytes"] == round(2000.0 * 1024 * 1.2)      # mean of the two dispatches, scaled
    assert k1["write_bytes"] == 500 * 1024
    assert k1["bytes_per_launch"] == k1["fetch_bytes"] + k1["write_bytes"]
    assert rec["kernels"]["gemm2_residual"]["fetch_bytes"] == round(600.0 * 1024 * 1.2)
    assert set(rec["kernels"]) == {"gemm1_gelu", "gemm2_residual"}
    assert rec["gemm_source_sha256_16"] == counters.gemm_hash()
    json.dumps(rec)


def test_committed_record_is_well_formed():
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles",
                        "traffic_counters.json")
    with open(path) as f:
        rec = json.load(f)
    assert "request" in rec["method"]
    assert {"gemm1_gelu", "gemm2_residual"} <= set(rec["kernels"])
    for k, e in rec["kernels"].items():
        assert abs(e["bytes_per_launch"] - e["read_bytes"] - e["write_bytes"]) <= 1
        assert e["read_bytes"] > 0 and e["write_bytes"] > 0


def test_mfma_utilisation_arithmetic(tmp_path):
    """Clock = GRBM_GUI_ACTIVE / XCCs / duration; busy = MFMA busy cycles / (SIMDs x cycles);
    FLOPs = 512 x MOPS.  One GPU agent with 4 SIMDs on 2 XCCs, two dispatches of GEMM1."""
    with open(tmp_path / "a.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Agent_Type", "Simd_Count", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Agent_Type": "CPU", "Simd_Count": 0, "Num_Xcc": 0})
        w.writerow({"Agent_Type": "GPU", "Simd_Count": 4, "Num_Xcc": 2})
    g1 = "void rmx::(anonymous namespace)::gemm_bf16_mfma<0, true, false, false>(rmx::GemmArgs)"
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(tmp_path / "c.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for disp, (gui, busy, start, end) in enumerate([(2000.0, 2000.0, 100, 600), (4000.0, 1000.0, 0, 1000)]):
            for name, val in (("GRBM_GUI_ACTIVE", gui), ("SQ_VALU_MFMA_BUSY_CYCLES", busy),
                              ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0)):
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": g1, "Counter_Name": name, "Counter_Value": val,
                            "Start_Timestamp": start, "End_Timestamp": end})
            w.writerow({"Dispatch_Id": 9, "Kernel_Name": "other", "Counter_Name": "GRBM_GUI_ACTIVE",
                        "Counter_Value": 1.0, "Start_Timestamp": 0, "End_Timestamp": 1})
    u = counters.mfma_utilisation(str(tmp_path / "c.csv"), str(tmp_path / "a.csv"))
    assert set(u) == {"gemm1_gelu"}
    e = u["gemm1_gelu"]
    assert e["dispatches"] == 2
    # dispatch 0: 1000 cycles in 500 ns = 2 GHz, busy 2000 / (4 x 1000) = 0.5, 512000 FLOP / 500 ns
    # dispatch 1: 2000 cycles in 1000 ns = 2 GHz, busy 1000 / (4 x 2000) = 0.125, 512000 / 1000 ns
    assert abs(e["clock_ghz"] - 2.0) < 1e-12
    assert abs(e["mfma_busy"] - (0.5 + 0.125) / 2) < 1e-12
    assert abs(e["ms"] - (500 + 1000) / 2 / 1e6) < 1e-15
    assert abs(e["tflops"] - (512000 / 500 + 512000 / 1000) / 2 / 1e3) < 1e-9


def test_request_record_prices_each_request_by_its_size(tmp_path):
    """Bytes per dispatch are 32, 64 and 128 per read request of that size and 64 per 64-byte
    write, 32 per other write; no scale factor enters."""
    g1 = "void rmx::(anonymous namespace)::gemm_bf16_mfma_n192<0>(rmx::GemmArgs)"
    g2 = "void rmx::(anonymous namespace)::gemm_bf16_mfma_m64<1, true, 256>(rmx::GemmArgs)"
    rows = "void rmx::(anonymous namespace)::rows_kernel<rmx::bf16_t, 8, 3, 1, false>(rmx::RowsArgs)"
    rd = []
    for k, (a, b, c) in ((g1, (10.0, 20.0, 1000.0)), (g1, (30.0, 40.0, 3000.0)), (g2, (0.0, 0.0, 500.0)),
                         (rows, (0.0, 2.0, 64.0))):
        rd += [(k, "TCC_EA0_RDREQ_32B_sum", a), (k, "TCC_EA0_RDREQ_64B_sum", b), (k, "TCC_EA0_RDREQ_128B_sum", c),
               (k, "TCC_EA0_RDREQ_sum", a + b + c)]
    wr = []
    for k, (n, n64) in ((g1, (300.0, 200.0)), (g1, (300.0, 200.0)), (g2, (50.0, 50.0)), (rows, (8.0, 8.0))):
        wr += [(k, "TCC_EA0_WRREQ_sum", n), (k, "TCC_EA0_WRREQ_64B_sum", n64)]
    _write(tmp_path / "r.csv", rd)
    _write(tmp_path / "w.csv", wr)
    rec = counters.build_request_record(str(tmp_path / "r.csv"), str(tmp_path / "w.csv"), "w B=2")
    k1 = rec["kernels"]["gemm1_gelu"]
    assert k1["read_bytes"] == 32 * 20 + 64 * 30 + 128 * 2000      # means of the two dispatches
    assert k1["write_bytes"] == 64 * 200 + 32 * 100
    assert k1["bytes_per_launch"] == k1["read_bytes"] + k1["write_bytes"] and k1["dispatches"] == [2, 2]
    assert rec["kernels"]["gemm2_residual"]["read_bytes"] == 128 * 500
    assert rec["kernels"]["rows_ln2_mix_ln1"]["read_bytes"] == 64 * 2 + 128 * 64
    assert rec["gemm_source_sha256_16"] == counters.gemm_hash()


def test_kernel_stats_table_from_a_results_database(tmp_path):
    import sqlite3
    db = tmp_path / "run_results.db"
    con = sqlite3.connect(db)
    con.execute("create table top_kernels (name text, total_calls int, total_duration real, average real, "
                "percentage real)")
    con.executemany("insert into top_kernels values (?, ?, ?, ?, ?)",
                    [("a", 2, 100.0, 50.0, 10.0), ("b", 4, 900.0, 225.0, 90.0)])
    con.execute("create table kernels (name text, duration real)")
    con.executemany("insert into kernels values (?, ?)", [("a", 40e3), ("a", 60e3), ("b", 200e3), ("b", 250e3)])
    con.commit()
    con.close()
    rows = counters.kernel_stats(str(db))
    assert [r[0] for r in rows] == ["b", "a"] and rows[0][3] == 225.0
    assert rows[1][5:] == (40.0, 60.0) and rows[0][5:] == (200.0, 250.0)
