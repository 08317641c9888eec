"""Host-side parts of bench.py that run without a GPU: the CPU-oracle baseline record and
the one-GPU guard."""
import json
import os
import subprocess
import sys

import bench
from rankmixer_block_forward_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_baseline_record():
    rec = bench.cpu_baseline(synth.TINY, 32)
    assert rec["kind"] == "oracle" and rec["unit"] == "samples/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert rec["logical_cpus"] == os.cpu_count()
    assert "32 samples of tiny" in rec["sample"] and "median of 3 runs" in rec["sample"]
    one = rec["single_thread"]
    assert one["value"] > 0 and one["sample"].startswith("2 samples, one BLAS thread, median of 3 runs")


def test_mxfp8_byte_counts():
    """The roofline's algorithmic bytes take the operand width of the variant: MXFP8 moves
    33/32 bytes per operand value (code plus a scale per 32) where bf16 moves 2."""
    cfg = synth.B1
    B = 64
    f, b_bf16 = bench.gemm_counts(cfg, B)["gemm1_gelu"]
    _, b_mx = bench.gemm_counts(cfg, B, mxfp8=True)["gemm1_gelu"]
    T, D, kD = cfg.T, cfg.D, cfg.kD
    assert f == 2.0 * B * T * D * kD
    assert b_bf16 == 2.0 * (T * D * kD + B * T * D + B * T * kD)
    assert abs(b_mx - 33.0 / 32.0 * (T * D * kD + B * T * D + B * T * kD)) < 1.0
    _, g2_mx = bench.gemm_counts(cfg, B, mxfp8=True)["gemm2_residual"]
    assert abs(g2_mx - (33.0 / 32.0 * (T * kD * D + B * T * kD) + 2.0 * B * T * D + 4.0 * B * T * D)) < 1.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
