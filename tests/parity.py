"""Helpers of the GPU parity tests: run the HIP path and the fp64 oracle on the same
seeded inputs and measure the difference.

Tolerances (from the build's correctness requirements): Token Mixing bit-exact; fp32
paths rel-L2 <= 1e-5; bf16 paths rel-L2 <= 1e-2 and max-abs <= 5e-2 on the post-LN
tensors (X_L) and on the pooled output.
"""
import numpy as np

import oracle

FP32_REL_L2 = 1e-5
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 5e-2


def rel_l2(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(y, ref):
    return float(np.max(np.abs(np.asarray(y, dtype=np.float64) - np.asarray(ref, dtype=np.float64))))


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float32).numpy()


def sample_rows(B, n, seed=0):
    """n sample indices spread over [0, B): always the first and last, the rest seeded."""
    if n >= B:
        return np.arange(B)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, B - 1), size=max(0, n - 2), replace=False)
    return np.unique(np.concatenate([[0, B - 1], mid]))


def run_gpu(cfg, inp, with_xl=True, handle=None, packed=False):
    """Forward of synth inputs through the library; returns (o, X_L) as float32 arrays.
    packed: run on weights prepared with rmx_pack_weights (W1/W2 then not passed)."""
    import torch
    import rankmixer_block_forward_amd as rmx
    X, w = rmx.upload(inp)
    h = handle or rmx.Handle.for_config(cfg, max_batch=X.shape[0])
    try:
        if packed:
            w = dict(w, packed=h.pack_weights(w))
            del w["W1"], w["W2"]
        out = torch.full((X.shape[0], cfg.D), float("nan"), dtype=torch.float32, device=X.device)
        xl = torch.full_like(X, float("nan")) if with_xl else None
        h.forward(X, w, out=out, xl_out=xl)
        torch.cuda.synchronize()
        return to_np(out), (to_np(xl) if with_xl else None)
    finally:
        if handle is None:
            h.close()


def run_oracle(cfg, inp, rows=None):
    X = inp.X if rows is None else inp.X[rows]
    o, XL, _ = oracle.forward(X, inp.layers(), cfg.eps)
    return o, XL


def check(cfg, o, xl, o_ref, xl_ref, label=""):
    """Asserts the tolerance of cfg.dtype; returns the measured errors."""
    err = {"o_rel_l2": rel_l2(o, o_ref), "o_max_abs": max_abs(o, o_ref)}
    if xl is not None:
        err.update(xl_rel_l2=rel_l2(xl, xl_ref), xl_max_abs=max_abs(xl, xl_ref))
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    if cfg.dtype == "fp32":
        assert err["o_rel_l2"] <= FP32_REL_L2, f"{label}: {err}"
        if xl is not None:
            assert err["xl_rel_l2"] <= FP32_REL_L2, f"{label}: {err}"
    else:
        assert err["o_rel_l2"] <= BF16_REL_L2 and err["o_max_abs"] <= BF16_MAX_ABS, f"{label}: {err}"
        if xl is not None:
            assert err["xl_rel_l2"] <= BF16_REL_L2 and err["xl_max_abs"] <= BF16_MAX_ABS, f"{label}: {err}"
    print(f"{label}: {err}", flush=True)
    return err
