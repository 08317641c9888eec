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
    assert "32 samples of tiny" in rec["sample"]
    one = rec["single_thread"]
    assert one["value"] > 0 and one["sample"].startswith("2 samples, one BLAS thread")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
