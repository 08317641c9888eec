"""Benchmark of the RankMixer block forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--batch B] [--workload NAME] [--sweep]

A step is one forward pass of the whole hot path (L blocks of mixing + LayerNorm +
per-token FFN + LayerNorm, then the mean pool) over one batch of synthetic input that is
already resident in HBM.  Prints ONE JSON line: samples/s of the RankMixer-1B shape
(T=32, D=1536, k=4, L=2, bf16, B=2048), its TFLOP/s (GEMM FLOPs, 4 k L T D^2 per sample)
and fraction of the bf16 dense MFMA peak, the roofline of the dominant kernel (timed
with HIP events on the stream it runs on), and the fp64 CPU oracle timed on a bounded
sample on this host's cores.  --sweep prints one line per serving batch size instead.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "samples/sec + achieved TFLOP/s (% bf16 MFMA peak) for RankMixer-1B block fwd"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="rankmixer-1b")
    p.add_argument("--batch", type=int, default=None)
    p.add_argument("--sweep", action="store_true", help="one line per serving batch size")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-samples", type=int, default=768)
    p.add_argument("--routing-comparison", action="store_true",
                   help="Token Mixing versus the self-attention comparator at the 100M and 1B shapes")
    p.add_argument("--mxfp8", action="store_true",
                   help="the MXFP8 inference variant (weights prepared with rmx_pack_weights_mxfp8)")
    p.add_argument("--backward", action="store_true",
                   help="time one training step's compute instead: forward keeping activations + backward")
    p.add_argument("--tokenize", action="store_true",
                   help="time the tokenisation projection (rmx_tokenize) at the 1B input shape "
                        "(B x [T*d] -> B x T x D, d = 512) and print its line instead")
    p.add_argument("--library-reference", action="store_true",
                   help="time the vendor library's bf16 GEMM (torch.mm / torch.bmm on contiguous "
                        "operands) at reference shapes and at the two grouped-GEMM shapes, one JSON "
                        "line each, for scale; no RankMixer work")
    p.add_argument("--graph", action="store_true",
                   help="also time the same forward captured once in a HIP graph and replayed "
                        "(torch.cuda.CUDAGraph on the caller's stream): adds a hip_graph object")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="after the timed region, run a plain streaming kernel (torch.neg over 1 GiB "
                        "of fp32) three times on cold sources: reference dispatches of known bytes "
                        "for the memory-traffic counters")
    return p.parse_args()


def gemm_counts(cfg, B, mxfp8=False):
    """Algorithmic FLOPs and HBM bytes of one launch of each grouped GEMM.

    GEMM1: S[T,B,D] x W1[T,D,kD] -> H[T,B,kD];  GEMM2: H x W2[T,kD,D] + S -> Y[T,B,D] fp32.
    Bytes: weights once + activations read once + output written once.  Operands of the
    products take 2 B per value in bf16; in MXFP8 1 B per code plus one scale byte per 32
    values (33/32 B), while the residual S stays bf16 and Y fp32."""
    T, D, kD = cfg.T, cfg.D, cfg.kD
    op = 33.0 / 32.0 if mxfp8 else 2.0
    flops = 2.0 * B * T * D * kD
    w = op * T * D * kD
    g1 = w + op * B * T * D + op * B * T * kD
    g2 = w + op * B * T * kD + 2.0 * B * T * D + 4.0 * B * T * D
    return {"gemm1_gelu": (flops, g1), "gemm2_residual": (flops, g2)}


def traffic_for(kernel, cfg, B):
    """Per-launch HBM bytes measured with rocprofv3 counters, if taken on the current
    kernel source at this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    from rankmixer_block_forward_amd import counters
    if rec.get("gemm_source_sha256_16") != counters.gemm_hash():
        return None
    entry = rec.get("kernels", {}).get(kernel)
    if not entry or entry.get("workload") != f"{cfg.name} B={B}":
        return None
    return entry.get("bytes_per_launch")


def moe_active_flops(h, X, w, cfg, B):
    """GEMM FLOPs of one Sparse-MoE forward counted on active experts only: per active
    (sample, token, expert) 2 * (D * h + h * D), plus the router's 2 * D * E per (sample,
    token); the activity pattern is read from the gates of one forward."""
    import torch
    gates = torch.empty((cfg.L, B, cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    h.forward(X, w, gate_out=gates)
    torch.cuda.synchronize()
    active = int((gates > 0).sum().item())
    flops = active * 4.0 * cfg.D * cfg.moe_hidden + cfg.L * B * cfg.T * 2.0 * cfg.D * cfg.E
    return flops, active / gates.numel()


def time_forward(cfg, B, steps, warmup, calibrate_copy=False, mxfp8=False, prepare=True):
    import torch
    import rankmixer_block_forward_amd as rmx
    from rankmixer_block_forward_amd import synth

    t0 = time.time()
    inp = synth.make_inputs(cfg.with_(B=B), seed=0)
    X, w = rmx.upload(inp)
    del inp
    print(f"[bench] inputs {cfg.name} B={B} generated and resident in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)
    h = rmx.Handle.for_config(cfg, max_batch=B)
    if mxfp8:
        # weights quantized once to MXFP8 (model-load work, outside the timed region)
        w["packed_mxfp8"] = h.pack_weights_mxfp8(w)
        torch.cuda.synchronize()
    elif prepare and h.packed_weights_bytes() > 0:
        # weights prepared once for the matrix cores (model-load work, outside the timed region)
        w["packed"] = h.pack_weights(w)
        torch.cuda.synchronize()
    out = torch.empty((B, cfg.D), dtype=torch.float32, device="cuda")
    moe = moe_active_flops(h, X, w, cfg, B) if cfg.E > 0 else None
    calib = []
    if calibrate_copy:
        # three 1 GiB fp32 sources, written now and cold (out of the L2 and the memory-side
        # cache) by the time a plain streaming kernel (torch.neg) reads each once and writes
        # 1 GiB after the timed region: reference dispatches of known bytes for the counters
        n = (1 << 30) // 4
        calib = [(torch.zeros(n, dtype=torch.float32, device="cuda"),
                  torch.empty(n, dtype=torch.float32, device="cuda")) for _ in range(3)]
    for _ in range(warmup):
        h.forward(X, w, out=out)
    torch.cuda.synchronize()
    # the timed region: the production launch sequence, nothing recorded between launches
    t0 = time.perf_counter()
    for _ in range(steps):
        h.forward(X, w, out=out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # then the same steps again with a pair of HIP events around every launch (on the stream
    # the kernels run on): the per-kernel durations of the roofline and the breakdown
    h.profile_reset()
    h.profile_enable(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        h.forward(X, w, out=out)
    torch.cuda.synchronize()
    prof_elapsed = time.perf_counter() - t1
    h.profile_enable(False)
    prof = h.profile_read()
    prof["_profiled_ms_per_step"] = prof_elapsed / steps * 1e3
    assert torch.isfinite(out).all().item(), "non-finite output"
    if calib:
        for src, dst in calib:
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] calibration copies: 3 x streaming negation of {calib[0][0].numel() * 4} bytes "
              f"read and written, cold sources", file=sys.stderr, flush=True)
        del calib
    h.close()
    return elapsed, prof, moe


def time_graph(cfg, B, steps, warmup, mxfp8=False):
    """The forward captured once into a HIP graph and replayed: wall time of `steps` replays
    after `warmup` replays (inputs resident, weights prepared as in time_forward)."""
    import torch
    import rankmixer_block_forward_amd as rmx
    from rankmixer_block_forward_amd import synth

    inp = synth.make_inputs(cfg.with_(B=B), seed=0)
    X, w = rmx.upload(inp)
    del inp
    h = rmx.Handle.for_config(cfg, max_batch=B)
    if mxfp8:
        w["packed_mxfp8"] = h.pack_weights_mxfp8(w)
    elif h.packed_weights_bytes() > 0:
        w["packed"] = h.pack_weights(w)
    out = torch.empty((B, cfg.D), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h.forward(X, w, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.forward(X, w, out=out)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert torch.isfinite(out).all().item(), "non-finite output"
    del g
    h.close()
    return elapsed


def roofline(cfg, B, prof, peak_tflops=PEAK_BF16_TFLOPS):
    counts = gemm_counts(cfg, B, mxfp8=peak_tflops == PEAK_FP8_TFLOPS)
    ridge = peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9)
    # dominant kernel: the grouped GEMM with the larger total time
    kern = max(counts, key=lambda k: prof.get(k, {}).get("total_ms", 0.0))
    flops, nbytes = counts[kern]
    avg_s = prof[kern]["avg_ms"] / 1e3
    mfma_bound = flops / nbytes > ridge
    traffic = traffic_for(kern, cfg, B) if peak_tflops == PEAK_BF16_TFLOPS else None
    if mfma_bound:
        achieved = flops / avg_s / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_tflops, "unit": "TFLOP/s",
             "frac": round(achieved / peak_tflops, 4)}
    else:
        achieved = nbytes / avg_s / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(achieved / PEAK_HBM_GBS, 4)}
    r["traffic"] = traffic
    r["kernel"] = kern
    r["avg_launch_ms"] = round(prof[kern]["avg_ms"], 4)
    r["algorithmic_flops_per_launch"] = flops
    r["algorithmic_bytes_per_launch"] = nbytes
    return r


def moe_roofline(cfg, B, prof, moe):
    """Roofline of the dominant Sparse-MoE kernel (the expert GEMM with the larger time),
    its FLOPs being half of the active expert FLOPs (each expert layer does D * h MACs)."""
    kern = max(("moe_ffn1", "moe_ffn2"), key=lambda k: prof.get(k, {}).get("total_ms", 0.0))
    active_flops = moe[0] - cfg.L * B * cfg.T * 2.0 * cfg.D * cfg.E
    flops = active_flops / 2.0 / cfg.L
    avg_s = prof[kern]["avg_ms"] / 1e3
    achieved = flops / avg_s / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": kern,
            "avg_launch_ms": round(prof[kern]["avg_ms"], 4), "algorithmic_flops_per_launch": flops}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, n, single_thread=True, repeats=3):
    """The fp64 oracle, as it stands, on n samples of the same workload with the BLAS
    threads the host gives it, the median of `repeats` timed runs over the same inputs; with
    single_thread, also on n/16 samples with one thread (median of as many runs)."""
    import numpy as np
    import oracle
    from rankmixer_block_forward_amd import synth
    threads = blas_threads()
    inp = synth.make_inputs(cfg.with_(B=n), seed=0)
    layers = inp.layers()

    def run(m):
        t0 = time.perf_counter()
        o, _, _ = oracle.forward(inp.X[:m], layers, cfg.eps)
        el = time.perf_counter() - t0
        assert np.isfinite(o).all()
        return el

    els = sorted(run(n) for _ in range(repeats))
    el = els[len(els) // 2]
    res = {"value": round(n / el, 3), "unit": "samples/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{n} samples of {cfg.name} (T={cfg.T}, D={cfg.D}, k={cfg.k}, L={cfg.L}), "
                     f"fp64 NumPy, median of {repeats} runs: " + ", ".join(f"{e:.1f}" for e in els) + " s",
           "cpu_model": cpu_model(), "logical_cpus": os.cpu_count()}
    if single_thread:
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:
            return res
        n1 = max(1, n // 16)
        with threadpool_limits(limits=1, user_api="blas"):
            els1 = sorted(run(n1) for _ in range(repeats))
        el1 = els1[len(els1) // 2]
        res["single_thread"] = {"value": round(n1 / el1, 3), "unit": "samples/s",
                                "sample": f"{n1} samples, one BLAS thread, median of {repeats} runs: "
                                          + ", ".join(f"{e:.1f}" for e in els1) + " s"}
    return res


def library_reference():
    """The platform library's bf16 GEMM at a few shapes (contiguous operands only)."""
    import torch
    torch.manual_seed(0)

    def timeit(f, n=10):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for n in (4096, 8192, 16384):
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        b = (torch.randn(n, n, device="cuda") / n ** 0.5).to(torch.bfloat16)
        ms = timeit(lambda: torch.mm(a, b))
        print(json.dumps({"library_gemm": f"mm {n}x{n}x{n}", "ms": round(ms, 4),
                          "tflops": round(2.0 * n ** 3 / ms / 1e9, 1)}), flush=True)
        del a, b
    G, M, D, kD = 32, 2048, 1536, 6144
    for name, (k, n) in (("GEMM1 shape", (D, kD)), ("GEMM2 shape", (kD, D))):
        # activations ~ N(0, 1), weights ~ N(0, 1/K): the workload's value ranges
        a = torch.randn(G, M, k, device="cuda", dtype=torch.bfloat16)
        b = (torch.randn(G, k, n, device="cuda") / k ** 0.5).to(torch.bfloat16).contiguous()
        ms = timeit(lambda: torch.bmm(a, b))
        print(json.dumps({"library_gemm": f"bmm {G}x({M}x{k})x({k}x{n}) {name}", "ms": round(ms, 4),
                          "tflops": round(2.0 * G * M * k * n / ms / 1e9, 1)}), flush=True)
        del a, b


def bench_tokenize(B, steps, warmup):
    """The tokenisation projection at the 1B input: E [B, T*d] -> X [B, T, D]."""
    import torch
    import rankmixer_block_forward_amd as rmx
    from rankmixer_block_forward_amd import synth
    T, D, d = synth.B1.T, synth.B1.D, synth.TOKENIZE_D
    ti = synth.make_tokenize_inputs(B, T, d, D, "bf16", seed=0)

    def dev(a):
        return torch.from_numpy(a).to("cuda").to(torch.bfloat16).contiguous()
    E, Wp, bp = dev(ti.E), dev(ti.Wp), dev(ti.bp)
    X = torch.empty((B, T, D), dtype=torch.bfloat16, device="cuda")
    for _ in range(warmup):
        rmx.tokenize(E, Wp, bp, X=X)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        rmx.tokenize(E, Wp, bp, X=X)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert torch.isfinite(X.float()).all().item()
    flops = 2.0 * B * T * d * D
    nbytes = 2.0 * (B * T * d + T * d * D + T * D + B * T * D)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / nbytes > ridge:
        ach = flops / (ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    else:
        ach = nbytes / (ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof.update(traffic=None, kernel="tokenize", avg_launch_ms=round(ms, 4),
                algorithmic_flops_per_launch=flops, algorithmic_bytes_per_launch=nbytes)
    print(json.dumps({
        "metric": "tokenisation projection: samples/s (concatenated embedding -> T tokens of D)",
        "value": round(B / (ms / 1e3), 1), "unit": "samples/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian embedding and random-init projections)",
        "config": {"workload": "rankmixer-1b-tokenize", "B": B, "T": T, "d": d, "D": D},
        "tflops": round(flops / (ms / 1e3) / 1e12, 2), "roofline": roof}), flush=True)


def bench_backward(cfg, B, steps, warmup, cpu_samples):
    """A step = rmx_block_forward_train + rmx_block_backward over one resident batch (the
    gradients of every parameter and of X for an upstream gradient of the pooled output).
    FLOPs per step: forward 4 k L T D^2 per sample, backward twice that (gradients of the
    activations and of the weights, two products each per block)."""
    import numpy as np
    import torch
    import rankmixer_block_forward_amd as rmx
    from rankmixer_block_forward_amd import synth
    t0 = time.time()
    inp = synth.make_inputs(cfg.with_(B=B), seed=0)
    X, w = rmx.upload(inp)
    del inp
    g = torch.from_numpy(synth.make_grad_out(B, cfg.D, seed=0)).cuda()
    print(f"[bench] inputs {cfg.name} B={B} generated and resident in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)
    h = rmx.Handle.for_config(cfg, max_batch=B)
    if h.packed_weights_bytes() > 0:
        # weights prepared once (model-load work): the training forward's products read them,
        # the backward reads W1 and W2
        w["packed"] = h.pack_weights(w)
        torch.cuda.synchronize()
    out, saved = h.forward_train(X, w)
    dX, grads = h.backward(X, w, saved, g)
    for _ in range(warmup):
        h.forward_train(X, w, out=out, saved=saved)
        h.backward(X, w, saved, g, dX=dX, grads=grads)
    torch.cuda.synchronize()
    h.profile_reset()
    h.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        h.forward_train(X, w, out=out, saved=saved)
        h.backward(X, w, saved, g, dX=dX, grads=grads)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    h.profile_enable(False)
    prof = h.profile_read()
    assert torch.isfinite(dX).all().item() and torch.isfinite(grads["W1"]).all().item()
    h.close()
    ms = elapsed / steps * 1e3
    fwd_flops = B * 4.0 * cfg.k * cfg.L * cfg.T * cfg.D * cfg.D
    flops = 3.0 * fwd_flops
    per_launch = 2.0 * B * cfg.T * cfg.D * cfg.k * cfg.D
    bwd = ("bwd_gemm_dU", "bwd_gemm_dS", "bwd_gemm_dW1", "bwd_gemm_dW2")
    kern = max(bwd, key=lambda k: prof.get(k, {}).get("total_ms", 0.0))
    ach = per_launch / (prof[kern]["avg_ms"] / 1e3) / 1e12
    roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": kern,
            "avg_launch_ms": round(prof[kern]["avg_ms"], 4), "algorithmic_flops_per_launch": per_launch}
    line = {
        "metric": "training step compute (forward keeping activations + backward): samples/s and TFLOP/s",
        "value": round(B / (ms / 1e3), 1), "unit": "samples/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian inputs, random-init weights, Gaussian gradient of the pooled output)",
        "config": {"workload": cfg.name + "-train", "B": B, "T": cfg.T, "H": cfg.T, "D": cfg.D, "k": cfg.k,
                   "L": cfg.L, "parallelism": "single GPU"},
        "tflops": round(flops / (ms / 1e3) / 1e12, 2),
        "frac_bf16_peak": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernels_ms_per_step": {k: round(v["total_ms"] / steps, 4) for k, v in prof.items() if not k.startswith("_")},
        "roofline": roof,
    }
    if cpu_samples:
        import oracle
        n = max(1, cpu_samples // 8)
        inp = synth.make_inputs(cfg.with_(B=n), seed=0)
        go = synth.make_grad_out(n, cfg.D, seed=0)
        t0 = time.perf_counter()
        o, _, _ = oracle.forward(inp.X, inp.layers(), cfg.eps)
        dXo, _ = oracle.backward(inp.X, inp.layers(), go, cfg.eps)
        el = time.perf_counter() - t0
        assert np.isfinite(dXo).all()
        line["cpu_baseline"] = {"value": round(n / el, 3), "unit": "samples/s", "cores": int(blas_threads()),
                                "kind": "oracle", "sample": f"{n} samples of {cfg.name}: fp64 forward + "
                                                            f"backward, {el:.1f} s"}
    print(json.dumps(line), flush=True)


def bench_routing(steps, warmup):
    """The pages' routing ablation on this harness: the same blocks with Token Mixing and with
    the self-attention comparator, both on the row-major weights (the comparator has no
    prepared-weights path), at the 100M shape (where the pages ran it) and the 1B shape."""
    from rankmixer_block_forward_amd import synth
    for mix in (synth.M100, synth.B1):
        att = mix.with_(name=mix.name + "-attention", routing="attention")
        T, D, k, L = mix.T, mix.D, mix.k, mix.L
        t_mix, prof_mix, _ = time_forward(mix, mix.B, steps, warmup, prepare=False)
        t_att, prof_att, _ = time_forward(att, mix.B, steps, warmup, prepare=False)
        f_mix = 4.0 * k * L * T * D * D                          # per sample
        f_att = f_mix + L * (6.0 * T * D * D + 4.0 * T * T * D)  # + Q, K, V and the scores / sum
        p_mix = L * 2.0 * T * D * k * D                          # per-token FFN weights
        p_att = p_mix + L * 3.0 * D * D
        ms_mix, ms_att = t_mix / steps * 1e3, t_att / steps * 1e3
        print(json.dumps({
            "metric": "routing comparison: Token Mixing vs self-attention, samples/s of each",
            "value": round(mix.B / (ms_att / 1e3), 1), "unit": "samples/s (attention routing)", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "higher_is_better": True, "vs_baseline": None, "dtype": mix.dtype,
            "data": "synthetic (seeded Gaussian inputs and random-init weights)",
            "config": {"workload": mix.name + "-routing", "B": mix.B, "T": T, "D": D, "k": k, "L": L},
            "mix": {"samples_per_s": round(mix.B / (ms_mix / 1e3), 1), "ms_per_step": round(ms_mix, 4),
                    "flops_per_sample": f_mix, "ffn_params": p_mix,
                    "kernels_ms_per_step": {n: round(v["total_ms"] / steps, 4) for n, v in prof_mix.items()
                                            if not n.startswith("_")}},
            "attention": {"samples_per_s": round(mix.B / (ms_att / 1e3), 1), "ms_per_step": round(ms_att, 4),
                          "flops_per_sample": f_att, "params": p_att,
                          "kernels_ms_per_step": {n: round(v["total_ms"] / steps, 4) for n, v in prof_att.items()
                                                  if not n.startswith("_")}},
            "flops_ratio": round(f_att / f_mix, 4), "param_ratio": round(p_att / p_mix, 4),
            "time_ratio": round(ms_att / ms_mix, 4)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.library_reference:
        library_reference()
        return
    if args.tokenize:
        bench_tokenize(args.batch or 2048, args.steps, args.warmup)
        return
    from rankmixer_block_forward_amd import synth
    cfg = synth.CONFIGS[args.workload]
    if args.routing_comparison:
        bench_routing(args.steps, args.warmup)
        return
    if args.backward:
        bench_backward(cfg, args.batch or cfg.B, args.steps, args.warmup,
                       0 if args.no_cpu_baseline else args.cpu_samples)
        return
    batches = list(synth.SWEEP_BATCHES) if args.sweep else [args.batch or cfg.B]
    if args.sweep:
        cfg = synth.SWEEP
    for B in batches:
        elapsed, prof, moe = time_forward(cfg, B, args.steps, args.warmup, args.calibrate_copy, args.mxfp8)
        ms = elapsed / args.steps * 1e3
        flops = B * 4.0 * cfg.k * cfg.L * cfg.T * cfg.D * cfg.D if moe is None else moe[0]
        tflops = flops / (ms / 1e3) / 1e12
        line = {
            "metric": METRIC,
            "value": round(B / (ms / 1e3), 1),
            "unit": "samples/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": cfg.dtype,
            "data": "synthetic (seeded Gaussian inputs and random-init weights at the workload's shapes)",
            "config": {"workload": cfg.name, "B": B, "T": cfg.T, "H": cfg.T, "D": cfg.D, "k": cfg.k,
                       "L": cfg.L, "zeroed_token_rows": cfg.zero_frac, "parallelism": "single GPU"},
            "tflops": round(tflops, 2),
            "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "kernels_ms_per_step": {k: round(v["total_ms"] / args.steps, 4) for k, v in prof.items()
                                    if not k.startswith("_")},
            "profiled_ms_per_step": round(prof["_profiled_ms_per_step"], 4),
            "roofline": (moe_roofline(cfg, B, prof, moe) if moe is not None else
                         roofline(cfg, B, prof, PEAK_FP8_TFLOPS if args.mxfp8 else PEAK_BF16_TFLOPS)),
        }
        if args.mxfp8:
            line["metric"] = METRIC.replace("block fwd", "block fwd, MXFP8 inference variant")
            line["dtype"] = "mxfp8 (E4M3 operands, E8M0 scales per 32; bf16 activations)"
            line["config"]["workload"] = cfg.name + "-mxfp8"
            line["frac_fp8_peak"] = round(tflops / PEAK_FP8_TFLOPS, 4)
        if moe is not None:
            line["config"].update(experts=cfg.E, expert_hidden=cfg.moe_hidden, active_fraction=round(moe[1], 4))
        if args.graph and moe is None:
            g_el = time_graph(cfg, B, args.steps, args.warmup, args.mxfp8)
            g_ms = g_el / args.steps * 1e3
            line["hip_graph"] = {"value": round(B / (g_ms / 1e3), 1), "unit": "samples/s",
                                 "ms_per_step": round(g_ms, 4)}
        if not args.sweep and not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_samples)
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
