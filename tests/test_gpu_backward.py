"""GPU parity of the block backward (rmx_block_forward_train + rmx_block_backward) against
the fp64 backward oracle, through the C ABI.

Tolerances.  fp32 path: rel-L2 <= 1e-5 on every gradient tensor (the forward's fp32
requirement).  bf16 path: rel-L2 <= 1e-2 and max-abs <= 5e-2 * max|ref| on every gradient
tensor.  Derivation of the bf16 bound: besides the forward's bf16 roundings (S, U, H),
the backward rounds two operands to bf16, the gradients of the pre-LN2 rows and of the
pre-activations; each rounding is a relative error of at most 2^-9 per element (RMS
2^-9 / sqrt 3 = 1.1e-3) that enters each product once, and per block a gradient passes
through at most three such products, so the expected relative error is a few 1e-3; 1e-2
keeps a margin of about 2 over the largest measured case.
"""
import numpy as np
import pytest

import oracle
from rankmixer_block_forward_amd import synth
from tests.parity import rel_l2, sample_rows, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FP32_TOL = 1e-5
BF16_REL_L2 = 1e-2
BF16_MAX_ABS_FRAC = 5e-2
NAMES = ("W1", "b1", "W2", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")


def _rmx():
    import rankmixer_block_forward_amd as rmx
    rmx.load_library()
    return rmx


def _gpu_backward(cfg, inp, g_out, handle=None):
    """forward_train then backward on the GPU; returns (out, dX, grads) as float64 arrays."""
    rmx = _rmx()
    X, w = rmx.upload(inp)
    h = handle or rmx.Handle.for_config(cfg, max_batch=X.shape[0])
    try:
        out, saved = h.forward_train(X, w)
        g = torch.from_numpy(g_out).cuda()
        dX, grads = h.backward(X, w, saved, g)
        torch.cuda.synchronize()
        return (to_np(out).astype(np.float64), to_np(dX).astype(np.float64),
                {n: to_np(t).astype(np.float64) for n, t in grads.items()})
    finally:
        if handle is None:
            h.close()


def _oracle_backward(cfg, inp, g_out, rows=None):
    X = inp.X if rows is None else inp.X[rows]
    g = g_out if rows is None else g_out[rows]
    dX, per_block = oracle.backward(X, inp.layers(), g, cfg.eps)
    grads = {n: np.stack([p[n] for p in per_block]) for n in NAMES}
    return dX, grads


def _check(cfg, got, ref, label):
    errs = {}
    for name in ref:
        y, r = got[name], ref[name]
        assert y.shape == r.shape, (label, name, y.shape, r.shape)
        assert np.isfinite(y).all(), f"{label}: {name} not finite"
        e = rel_l2(y, r)
        errs[name] = e
        if cfg.dtype == "fp32":
            assert e <= FP32_TOL, f"{label}: {name} rel-L2 {e:.3e}"
        else:
            ma = float(np.max(np.abs(y - r)))
            assert e <= BF16_REL_L2, f"{label}: {name} rel-L2 {e:.3e}"
            assert ma <= BF16_MAX_ABS_FRAC * float(np.max(np.abs(r))), f"{label}: {name} max-abs {ma:.3e}"
    print(label, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    return errs


CASES = [
    # name, cfg: the scalar row path and generic products (fp32), the vectorized fp32 path,
    # bf16 on the matrix cores with ragged rows and a ragged K tail of the weight-gradient
    # products, biases and LayerNorm affine parameters away from 1 / 0, a shape the
    # row-tile products do not take (K = D = 40), and a single sample.
    synth.TINY.with_(name="bwd-tiny-fp32", B=8),
    synth.Config("bwd-fp32-vec", B=6, T=4, D=32, k=2, L=2, dtype="fp32", bias_std=0.1),
    synth.Config("bwd-bf16-48", B=48, T=4, D=256, k=4, L=2, bias_std=0.05),
    synth.Config("bwd-bf16-300", B=300, T=8, D=256, k=2, L=2, bias_std=0.05),
    synth.Config("bwd-bf16-generic", B=50, T=5, D=40, k=2, L=2, bias_std=0.05),
    synth.Config("bwd-bf16-one", B=1, T=4, D=256, k=4, L=1),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_backward_matches_oracle(cfg):
    print(f"case {cfg.name}", flush=True)
    inp = synth.make_inputs(cfg, seed=3)
    g_out = synth.make_grad_out(cfg.B, cfg.D, seed=3)
    _, dX, grads = _gpu_backward(cfg, inp, g_out)
    rdX, rgrads = _oracle_backward(cfg, inp, g_out)
    _check(cfg, dict(grads, dX=dX), dict(rgrads, dX=rdX), cfg.name)


@pytest.mark.parametrize("cfg", [CASES[1], CASES[3]], ids=["fp32", "bf16"])
def test_forward_train_output_is_the_forward_output(cfg):
    """The training forward computes the same out as rmx_block_forward, bit for bit."""
    rmx = _rmx()
    inp = synth.make_inputs(cfg, seed=4)
    X, w = rmx.upload(inp)
    with rmx.Handle.for_config(cfg) as h:
        ref = h.forward(X, w)
        out, saved = h.forward_train(X, w)
        torch.cuda.synchronize()
        assert saved.numel() >= h.saved_bytes(cfg.B) > 0
        assert torch.equal(out, ref)


@pytest.mark.parametrize("B,T,D,k,L", [
    (300, 4, 384, 4, 2),   # both products on 256 x 384 tiles from the prepared copy, ragged rows
    (129, 8, 384, 2, 1),   # one row past a tile
    (300, 4, 256, 3, 2),   # only GEMM1 (N = kD = 768) reads the prepared copy; GEMM2 (N = 256) W2
    (1, 2, 768, 4, 1),     # one sample
])
def test_forward_train_on_prepared_weights_same_bits(B, T, D, k, L):
    """The training forward given the prepared copy (its products read W^T packed and the saved
    S and H row-major, gathered into the packed LDS layout) writes the same out and the same
    saved activations, bit for bit, as on W1 and W2; the backward from either is the same."""
    rmx = _rmx()
    cfg = synth.Config("train-pk", B=B, T=T, D=D, k=k, L=L, dtype="bf16", bias_std=0.02)
    inp = synth.make_inputs(cfg, seed=B + D)
    X, w = rmx.upload(inp)
    g = torch.from_numpy(synth.make_grad_out(B, D, seed=B)).cuda()
    with rmx.Handle.for_config(cfg) as h:
        o1, s1 = h.forward_train(X, w)
        wp = dict(w, packed=h.pack_weights(w))
        o2, s2 = h.forward_train(X, wp)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
        dX1, g1 = h.backward(X, w, s1, g)
        dX2, g2 = h.backward(X, wp, s2, g)
        torch.cuda.synchronize()
        assert torch.equal(dX1, dX2) and all(torch.equal(g1[n], g2[n]) for n in g1)
        o3 = h.forward(X, wp)
        torch.cuda.synchronize()
        assert torch.equal(o1, o3)   # the inference forward on the prepared copy: the same bits


def test_backward_twice_is_deterministic_and_reuses_the_workspace():
    cfg = CASES[3]
    rmx = _rmx()
    inp = synth.make_inputs(cfg, seed=5)
    g_out = synth.make_grad_out(cfg.B, cfg.D, seed=5)
    with rmx.Handle.for_config(cfg) as h:
        a = _gpu_backward(cfg, inp, g_out, handle=h)
        b = _gpu_backward(cfg, inp, g_out, handle=h)
    np.testing.assert_array_equal(a[1], b[1])
    for n in NAMES:
        np.testing.assert_array_equal(a[2][n], b[2][n])


def test_smaller_batch_after_larger_on_one_handle():
    """B below max_batch: the saved layout and the workspace follow the call's B."""
    cfg = CASES[3]
    rmx = _rmx()
    small = cfg.with_(B=77)
    inp = synth.make_inputs(small, seed=6)
    g_out = synth.make_grad_out(small.B, small.D, seed=6)
    with rmx.Handle.for_config(cfg) as h:
        big = synth.make_inputs(cfg, seed=7)
        _gpu_backward(cfg, big, synth.make_grad_out(cfg.B, cfg.D, seed=7), handle=h)
        _, dX, grads = _gpu_backward(small, inp, g_out, handle=h)
    rdX, rgrads = _oracle_backward(small, inp, g_out)
    _check(small, dict(grads, dX=dX), dict(rgrads, dX=rdX), "B=77 after B=300")


def test_samples_without_gradient_get_exact_zeros():
    """Rows of g_out that are zero give exactly zero dX rows: nothing leaks across samples."""
    cfg = CASES[3]
    rows = [0, 17, 299]
    inp = synth.make_inputs(cfg, seed=8)
    g_out = synth.make_grad_out(cfg.B, cfg.D, seed=8, rows=rows)
    _, dX, grads = _gpu_backward(cfg, inp, g_out)
    others = np.setdiff1d(np.arange(cfg.B), rows)
    assert not dX[others].any()
    rdX, rgrads = _oracle_backward(cfg, inp, g_out, rows=rows)
    _check(cfg, dict(grads, dX=dX[rows]), dict(rgrads, dX=rdX), "three samples with gradient")


@pytest.mark.slow
def test_backward_1b_full_size_sampled():
    """RankMixer-1B at B = 2048: g_out is nonzero on 8 sampled rows only, so every gradient
    comes from those samples and the oracle computes all of them exactly from the 8; the
    other 2040 dX rows must be exactly zero.  The weight gradients are compared on four
    tokens per block (the oracle computes all 32)."""
    cfg = synth.B1.with_(bias_std=0.02)
    rows = sample_rows(cfg.B, 8, seed=9)
    inp = synth.make_inputs(cfg, seed=0)
    g_out = synth.make_grad_out(cfg.B, cfg.D, seed=9, rows=rows)
    rmx = _rmx()
    X, w = rmx.upload(inp)
    toks = [0, 7, 20, 31]
    with rmx.Handle.for_config(cfg) as h:
        # the training forward on the prepared copy (the benchmark's launch), which must give
        # the bits of the forward on W1 and W2
        wp = dict(w, packed=h.pack_weights(w))
        out, saved = h.forward_train(X, wp)
        out_rm, saved_rm = h.forward_train(X, w)
        torch.cuda.synchronize()
        assert torch.equal(out, out_rm) and torch.equal(saved, saved_rm)
        del saved_rm
        dX, grads = h.backward(X, wp, saved, torch.from_numpy(g_out).cuda())
        torch.cuda.synchronize()
        got = {n: to_np(t).astype(np.float64) for n, t in grads.items() if n not in ("W1", "W2")}
        got["W1"] = to_np(grads["W1"][:, toks]).astype(np.float64)
        got["W2"] = to_np(grads["W2"][:, toks]).astype(np.float64)
        dX = to_np(dX)
    del grads, saved
    others = np.setdiff1d(np.arange(cfg.B), rows)
    assert not dX[others].any()
    rdX, rgrads = _oracle_backward(cfg, inp, g_out, rows=rows)
    rgrads["W1"] = rgrads["W1"][:, toks]
    rgrads["W2"] = rgrads["W2"][:, toks]
    _check(cfg, dict(got, dX=dX[rows].astype(np.float64)), dict(rgrads, dX=rdX), "1B B=2048, 8 rows")


@pytest.mark.slow
def test_backward_1b_full_size_dx_of_sampled_rows():
    """RankMixer-1B at B = 2048 with every row of g_out nonzero: dX of a sample depends on
    that sample alone, so the oracle checks dX on 6 sampled rows; the parameter gradients
    are additive over samples, checked against the sum of two backward passes over
    complementary halves of g_out."""
    cfg = synth.B1
    rows = sample_rows(cfg.B, 6, seed=10)
    inp = synth.make_inputs(cfg, seed=0)
    g_out = synth.make_grad_out(cfg.B, cfg.D, seed=10)
    rmx = _rmx()
    X, w = rmx.upload(inp)
    half = np.arange(cfg.B) < cfg.B // 2
    with rmx.Handle.for_config(cfg) as h:
        _, saved = h.forward_train(X, w)
        g = torch.from_numpy(g_out).cuda()
        dX, full = h.backward(X, w, saved, g)
        dX = to_np(dX)
        _, ga = h.backward(X, w, saved, g * torch.from_numpy(half.astype(np.float32)).cuda()[:, None])
        _, gb = h.backward(X, w, saved, g * torch.from_numpy((~half).astype(np.float32)).cuda()[:, None])
        torch.cuda.synchronize()
        for n in ("b1", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b", "W2"):
            r = rel_l2(to_np(ga[n] + gb[n]), to_np(full[n]))
            assert r <= 1e-5, (n, r)
    rdX, _ = _oracle_backward(cfg.with_(B=len(rows)), _subset(inp, rows), g_out[rows])
    e = rel_l2(dX[rows], rdX)
    ma = float(np.max(np.abs(dX[rows] - rdX)))
    print("1B dX on sampled rows", e, ma, flush=True)
    assert e <= BF16_REL_L2 and ma <= BF16_MAX_ABS_FRAC * float(np.max(np.abs(rdX)))


def _subset(inp, rows):
    import dataclasses
    return dataclasses.replace(inp, X=inp.X[rows])


def test_backward_argument_errors():
    rmx = _rmx()
    from rankmixer_block_forward_amd.binding import RmxError, RMX_ERR_INVALID_ARG, RMX_ERR_UNSUPPORTED
    cfg = CASES[2]
    inp = synth.make_inputs(cfg, seed=11)
    X, w = rmx.upload(inp)
    g = torch.from_numpy(synth.make_grad_out(cfg.B, cfg.D, seed=11)).cuda()
    with rmx.Handle.for_config(cfg) as h:
        out, saved = h.forward_train(X, w)
        with pytest.raises(RmxError) as ei:       # saved buffer too small
            h.backward(X, w, saved[: saved.numel() // 2], g)
        assert ei.value.status == RMX_ERR_INVALID_ARG
        with pytest.raises(RmxError) as ei:       # training needs W1 and W2 beside prepared weights
            h.forward_train(X, dict(w, packed=h.pack_weights(w), W1=None))
        assert ei.value.status == RMX_ERR_INVALID_ARG
        dX = torch.empty((cfg.B, cfg.T, cfg.D), dtype=torch.float32, device="cuda")
        grads = {n: torch.empty(1, device="cuda") for n in NAMES}
        with pytest.raises(ValueError):           # binding checks gradient shapes
            h.backward(X, w, saved, g, dX=dX, grads=grads)
        torch.cuda.synchronize()
    moe = synth.Config("bwd-moe", B=16, T=4, D=256, k=4, L=1, E=2, moe_hidden=256)
    with rmx.Handle.for_config(moe) as h:
        assert h.saved_bytes(16) == 0
        minp = synth.make_inputs(moe, seed=12)
        MX, mw = rmx.upload(minp)
        with pytest.raises(RmxError) as ei:
            h.forward_train(MX, mw)
        assert ei.value.status == RMX_ERR_UNSUPPORTED
