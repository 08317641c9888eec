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


def sample_tiles(B, per_tile, tile=256, seed=0):
    """Sample indices stratified over the 256-row tiles of the products: the first and last
    row of every tile (the ragged edges) plus per_tile - 2 seeded rows inside it."""
    rng = np.random.default_rng(seed)
    picks = []
    for t0 in range(0, B, tile):
        t1 = min(B, t0 + tile)
        picks += [t0, t1 - 1]
        inner = np.arange(t0 + 1, t1 - 1)
        if len(inner):
            picks += rng.choice(inner, size=min(len(inner), max(0, per_tile - 2)), replace=False).tolist()
    return np.unique(np.array(picks, dtype=np.int64))


def check_moe_lists(lists, gates, tile=256):
    """Bit-exact check of the Sparse-MoE routing lists of every block against the gate values
    the same forward wrote: group gi = t*E + e lists exactly the samples b with
    gates[n, b, t, e] > 0, as token rows t*B + b in ascending b; the lists are concatenated in
    group order; row_gate holds the same fp32 gate bits; pos is the inverse map (-1 when
    inactive); tile_start counts the 256-row tiles of the groups cumulatively.
    lists: dict of numpy arrays as Handle.forward_moe_lists returns them; gates [L, B, T, E].
    Returns the per-block active fraction."""
    L, B, T, E = gates.shape
    G = T * E
    frac = []
    for n in range(L):
        gs, rows, rg = lists["group_start"][n], lists["rows"][n], lists["row_gate"][n]
        pos, ts = lists["pos"][n].reshape(G, B), lists["tile_start"][n]
        g = gates[n].transpose(1, 2, 0).reshape(G, B)           # [t*E + e, b]
        act = g > 0
        counts = act.sum(axis=1)
        assert gs[0] == 0 and np.array_equal(np.diff(gs), counts), f"block {n}: group offsets"
        want_ts = np.concatenate([[0], np.cumsum((counts + tile - 1) // tile)])
        assert np.array_equal(ts, want_ts), f"block {n}: tile table"
        for gi in range(G):
            b = np.nonzero(act[gi])[0]
            lo, hi = gs[gi], gs[gi + 1]
            t = gi // E
            assert np.array_equal(rows[lo:hi], t * B + b), f"block {n} group {gi}: row list"
            assert np.array_equal(rg[lo:hi].view(np.uint32), g[gi, b].astype(np.float32).view(np.uint32)), \
                f"block {n} group {gi}: gate values"
            want_pos = np.full(B, -1, dtype=np.int64)
            want_pos[b] = lo + np.arange(len(b))
            assert np.array_equal(pos[gi], want_pos), f"block {n} group {gi}: inverse map"
        frac.append(float(counts.sum()) / (G * B))
    return frac
