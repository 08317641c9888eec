"""The hand-computed index maps of the kernels (rankmixer_block_forward_amd/csrc/rmx_layout.h:
the packed bf16 and MXFP8 operand layouts, the gather of row-major rows into them, the
dense tile order and the Sparse-MoE tile table) built as host code with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, and run over whole buffers of the sizes
the library allocates: the tested shapes, the 100M and 1B workloads and the largest serving
batch (B = 16384).  tests/native/layout_check.cpp states what each check holds the map to.
"""
import math
import os
import shutil
import subprocess

import pytest

from rankmixer_block_forward_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rankmixer_block_forward_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "layout_check.cpp")

# (B, T, D, k) of the dense parity tests, then the workloads
DENSE = [(1, 4, 256, 4), (33, 8, 256, 4), (129, 8, 384, 2), (300, 4, 384, 4), (300, 8, 256, 2), (48, 4, 256, 4),
         (40, 4, 192, 4), (4, 4, 96, 2), (64, 2, 128, 4), (257, 2, 768, 4)]
WORKLOADS = [(synth.M100.B, synth.M100.T, synth.M100.D, synth.M100.k),
             (synth.B1.B, synth.B1.T, synth.B1.D, synth.B1.k),
             (16384, synth.B1.T, synth.B1.D, synth.B1.k)]
# (B, T, D, E, moe_hidden) of the Sparse-MoE parity tests and the 1B Sparse-MoE workload
MOE = [(100, 4, 64, 4, 64), (300, 2, 256, 8, 96), (1, 4, 64, 2, 32), (257, 8, 128, 3, 128), (700, 2, 384, 8, 1152),
       (synth.MOE.B, synth.MOE.T, synth.MOE.D, synth.MOE.E, synth.MOE.moe_hidden),
       (16384, synth.MOE.T, synth.MOE.D, synth.MOE.E, synth.MOE.moe_hidden)]


def _commands():
    pk, mx, tiles, span = set(), set(), set(), set()
    for B, T, D, k in DENSE + WORKLOADS:
        kD = k * D
        # A and W^T of both products, and the GELU output (the second product's A)
        for rows, K in ((B, D), (kD, D), (B, kD), (D, kD)):
            if K % 32 == 0:
                pk.add((rows, K))
            if K % 64 == 0:
                mx.add((rows, K))
        for N in (kD, D):
            for tm, tn in ((256, 256), (256, 384), (128, 384), (256, 192), (128, 192), (64, 256)):
                if N % tn == 0:
                    nMt = math.ceil(B / tm)
                    tiles.add((nMt, N // tn, T * nMt * (N // tn)))
        span.add((B, D))
        span.add((B, kD))
    cmds = [f"pk {r} {K}" for r, K in sorted(pk)] + [f"mx {r} {K}" for r, K in sorted(mx)]
    cmds += ["gather"] + [f"tiles {a} {b} {c}" for a, b, c in sorted(tiles)]
    for i, (B, T, D, E, h) in enumerate(MOE):
        G = T * E
        for N in (h, D):
            for tn in (256, 384):
                if N % tn == 0 or tn == 256:
                    nNt = math.ceil(N / tn)
                    for zero in (0, 40):
                        cmds.append(f"moe {G} {nNt} {B} {1000 + i} {zero} 256")
        span.add((T * B, D))     # the first product gathers S through the row lists
        span.add((B, h))         # the second reads a group's compacted hidden rows
    # edge cases: every group empty; one group; the largest table (1024 groups); a grid of
    # one workgroup per XCD
    cmds += ["moe 8 4 500 7 100 256", "moe 1 1 1 8 0 8", "moe 1024 16 600 9 30 256", "moe 64 3 2048 10 20 8"]
    cmds += [f"span {r} {K}" for r, K in sorted(span)]
    return cmds


@pytest.fixture(scope="module")
def layout_check(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("layout") / "layout_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-DRMX_HD=", "-I", CSRC, SRC, "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


def test_index_maps_under_address_sanitizer(layout_check):
    cmds = _commands()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([layout_check], input="\n".join(cmds) + "\n", capture_output=True, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-4000:] + r.stdout[-2000:]
    assert r.stdout.strip().splitlines()[-1] == f"{len(cmds)} checks passed"
    assert "runtime error" not in r.stderr, r.stderr[-4000:]

