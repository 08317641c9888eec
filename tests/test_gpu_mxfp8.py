"""GPU parity of the MXFP8 inference variant (weights prepared with rmx_pack_weights_mxfp8),
through the C ABI.

Two references, both fp64 oracles:
  * oracle.forward_mxfp8, the same computation with the same quantization points (OCP MX:
    E4M3 codes, a power-of-two scale per 32 values along K).  With one block the GPU path
    must match it at the bf16 bar (rel-L2 <= 1e-2, max-abs <= 5e-2 on X_L and on out): the
    GPU quantizes fp32 values (the oracle fp64 ones: a code moves only where a value sits
    within fp32 rounding of a boundary, or in GELU's far left tail where its fp32 erf is
    relatively coarse), adds the residual from S in bf16 and accumulates in fp32.  From the
    second block on, the block input is the first block's output stored in bf16 (relative
    step 2^-9) while the oracle keeps fp64; E4M3 codes are 2^-4 .. 2^-3 apart relatively, so
    about 2 % of the second block's codes of S and H land on the other side of a rounding
    boundary and move by one E4M3 step: ~1.3 % rel-L2 measured; the bar is then rel-L2
    <= 3e-2 and max-abs <= 0.2;
  * oracle.forward, the unquantized block: the variant departs from it by the format's own
    precision, measured at 4.3-4.6 % rel-L2 (max-abs 0.10-0.24 on X_L) on these shapes and on
    the 100M and 1B shapes with the fp64 oracles alone; the bar is rel-L2 <= 8e-2 and
    max-abs <= 0.5, about twice that.
"""
import numpy as np
import pytest

import oracle
from rankmixer_block_forward_amd import synth
from tests.parity import rel_l2, max_abs, sample_rows, sample_tiles, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U_REL, U_ABS = 8e-2, 0.5           # against the unquantized oracle


def q_bar(L):
    """(rel-L2, max-abs) bar against the quantized oracle for L blocks."""
    return (1e-2, 5e-2) if L == 1 else (3e-2, 0.2)


CASES = [
    # ragged rows, nonzero biases; two row tiles with a short second one; one sample; K with
    # an even number of 64-steps and N below one 256-column tile; an odd number of steps
    synth.Config("mx-48", B=48, T=4, D=256, k=4, L=2, bias_std=0.05),
    synth.Config("mx-300", B=300, T=8, D=256, k=2, L=2, bias_std=0.05),
    synth.Config("mx-one", B=1, T=4, D=256, k=4, L=1),
    synth.Config("mx-l1", B=200, T=8, D=256, k=4, L=1, bias_std=0.05),
    synth.Config("mx-d128", B=64, T=2, D=128, k=4, L=2),
    synth.Config("mx-d192", B=40, T=4, D=192, k=4, L=2, bias_std=0.05),
]


def _run(cfg, inp, handle=None):
    import rankmixer_block_forward_amd as rmx
    X, w = rmx.upload(inp)
    h = handle or rmx.Handle.for_config(cfg, max_batch=X.shape[0])
    try:
        packed = h.pack_weights_mxfp8(w)
        wm = {k: v for k, v in w.items() if k not in ("W1", "W2")}
        wm["packed_mxfp8"] = packed
        out = torch.full((X.shape[0], cfg.D), float("nan"), dtype=torch.float32, device="cuda")
        xl = torch.full_like(X, float("nan"))
        h.forward(X, wm, out=out, xl_out=xl)
        torch.cuda.synchronize()
        return to_np(out).astype(np.float64), to_np(xl).astype(np.float64)
    finally:
        if handle is None:
            h.close()


def _check(label, o, xl, ref_o, ref_xl, rel, ab):
    err = {"o": rel_l2(o, ref_o), "o_abs": max_abs(o, ref_o), "xl": rel_l2(xl, ref_xl), "xl_abs": max_abs(xl, ref_xl)}
    print(label, {k: f"{v:.3e}" for k, v in err.items()}, flush=True)
    assert np.isfinite(o).all() and np.isfinite(xl).all(), label
    assert err["o"] <= rel and err["xl"] <= rel and err["o_abs"] <= ab and err["xl_abs"] <= ab, (label, err)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_mxfp8_matches_quantized_oracle_and_unquantized_within_format_precision(cfg):
    print(f"case {cfg.name}", flush=True)
    inp = synth.make_inputs(cfg, seed=21)
    o, xl = _run(cfg, inp)
    qo, qxl = oracle.forward_mxfp8(inp.X, inp.layers(), cfg.eps)
    _check(cfg.name + " vs quantized oracle", o, xl, qo, qxl, *q_bar(cfg.L))
    uo, uxl, _ = oracle.forward(inp.X, inp.layers(), cfg.eps)
    _check(cfg.name + " vs unquantized oracle", o, xl, uo, uxl, U_REL, U_ABS)


def test_mxfp8_is_deterministic_and_weights_prepare_identically():
    import rankmixer_block_forward_amd as rmx
    cfg = CASES[1]
    inp = synth.make_inputs(cfg, seed=22)
    X, w = rmx.upload(inp)
    with rmx.Handle.for_config(cfg) as h:
        p1, p2 = h.pack_weights_mxfp8(w), h.pack_weights_mxfp8(w)
        torch.cuda.synchronize()
        assert torch.equal(p1, p2)
        a = _run(cfg, inp, handle=h)
        b = _run(cfg, inp, handle=h)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_mxfp8_100m_full_size_sampled_rows():
    """RankMixer-100M at B = 512 through the MXFP8 path; the quantized oracle on 12 sampled
    samples (rows are independent, so their outputs are exact in meaning)."""
    cfg = synth.M100
    inp = synth.make_inputs(cfg, seed=0)
    o, xl = _run(cfg, inp)
    rows = sample_rows(cfg.B, 12, seed=23)
    X = inp.X[rows]
    qo, qxl = oracle.forward_mxfp8(X, inp.layers(), cfg.eps)
    _check("100M vs quantized oracle", o[rows], xl[rows], qo, qxl, *q_bar(cfg.L))
    uo, uxl, _ = oracle.forward(X, inp.layers(), cfg.eps)
    _check("100M vs unquantized oracle", o[rows], xl[rows], uo, uxl, U_REL, U_ABS)


@pytest.mark.slow
def test_mxfp8_1b_full_size_sampled_rows():
    """RankMixer-1B at B = 2048 (the benchmark workload) through the MXFP8 path, against the
    quantized oracle (its 128 weight matrices quantized on the host's threads) on 32 samples
    stratified over the row tiles, and against the unquantized oracle on the same samples."""
    import os
    cfg = synth.B1
    inp = synth.make_inputs(cfg, seed=0)
    print("case MXFP8 1B B=2048", flush=True)
    o, xl = _run(cfg, inp)
    rows = sample_tiles(cfg.B, 4, seed=24)
    wq = oracle.quantize_weights(inp.layers(), workers=min(16, os.cpu_count() or 1))
    print("weights quantized by the oracle", flush=True)
    qo, qxl = oracle.forward_mxfp8(inp.X[rows], inp.layers(), cfg.eps, wq=wq)
    _check("1B vs quantized oracle", o[rows], xl[rows], qo, qxl, *q_bar(cfg.L))
    uo, uxl, _ = oracle.forward(inp.X[rows], inp.layers(), cfg.eps)
    _check("1B vs unquantized oracle", o[rows], xl[rows], uo, uxl, U_REL, U_ABS)


def test_mxfp8_rejected_where_unsupported():
    import rankmixer_block_forward_amd as rmx
    from rankmixer_block_forward_amd.binding import RmxError, RMX_ERR_UNSUPPORTED, RMX_ERR_INVALID_ARG
    for cfg in (synth.Config("mx-fp32", B=4, T=4, D=64, k=2, L=1, dtype="fp32"),
                synth.Config("mx-d96", B=4, T=4, D=96, k=2, L=1)):
        inp = synth.make_inputs(cfg, seed=25)
        X, w = rmx.upload(inp)
        with rmx.Handle.for_config(cfg) as h:
            assert h.packed_weights_mxfp8_bytes() == 0
            with pytest.raises(RmxError) as ei:
                h.pack_weights_mxfp8(w)
            assert ei.value.status == RMX_ERR_UNSUPPORTED
    cfg = CASES[0]
    inp = synth.make_inputs(cfg, seed=26)
    X, w = rmx.upload(inp)
    with rmx.Handle.for_config(cfg) as h:
        packed = h.pack_weights_mxfp8(w)
        with pytest.raises(RmxError) as ei:       # the training path reads W1 and W2
            h.forward_train(X, dict(w, packed_mxfp8=packed))
        assert ei.value.status == RMX_ERR_INVALID_ARG
        with pytest.raises(ValueError):           # the binding takes the prepared bytes as uint8
            h.forward(X, dict(w, packed_mxfp8=packed.view(torch.bfloat16)))
        torch.cuda.synchronize()
