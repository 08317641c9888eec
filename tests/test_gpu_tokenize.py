"""Parity of the tokenisation projection (rmx_tokenize) with the fp64 oracle, on the GPU.

X[b, t] = E[b, t*d:(t+1)*d] Wp[t] + bp[t] ("RankMixer" paper translation, section 3.2
eq (2); "UniMixer" translation, eq (9)).  Shapes cover the 256-row MFMA tiles, the
64-row tiles, the generic kernel (fp32, and bf16 with d not a multiple of 32), ragged
rows and columns, d = D, and the 1B input (sampled rows).  Tolerances as for the forward:
fp32 rel-L2 <= 1e-5; bf16 rel-L2 <= 1e-2 and max-abs <= 5e-2 (X is rounded to bf16).
"""
import numpy as np
import pytest

import oracle
from rankmixer_block_forward_amd import synth
from tests.parity import BF16_MAX_ABS, BF16_REL_L2, FP32_REL_L2, max_abs, rel_l2, sample_rows, to_np

pytestmark = pytest.mark.gpu


def _upload(ti, dtype):
    import torch
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def dev(a):
        return torch.from_numpy(a).to("cuda").to(dt).contiguous()
    return dev(ti.E), dev(ti.Wp), dev(ti.bp)


def _check(X, ref, dtype, what):
    r, m = rel_l2(X, ref), max_abs(X, ref)
    if dtype == "fp32":
        assert r <= FP32_REL_L2, f"{what}: rel-L2 {r:.3e}"
    else:
        assert r <= BF16_REL_L2 and m <= BF16_MAX_ABS, f"{what}: rel-L2 {r:.3e} max-abs {m:.3e}"


@pytest.mark.parametrize("B,T,d,D,dtype", [
    (7, 3, 8, 16, "fp32"),         # generic kernel, fp32
    (300, 4, 64, 256, "bf16"),     # 256-row tiles, ragged rows
    (33, 5, 96, 320, "bf16"),      # 64-row tiles, ragged columns, odd K-step count
    (65, 2, 40, 24, "bf16"),       # d not a multiple of 32: generic kernel in bf16
    (16, 4, 1536, 1536, "bf16"),   # d = D
])
def test_tokenize_shapes(B, T, d, D, dtype):
    import rankmixer_block_forward_amd as rmx
    ti = synth.make_tokenize_inputs(B, T, d, D, dtype, seed=B + d, bias_std=0.05)
    E, Wp, bp = _upload(ti, dtype)
    X = to_np(rmx.tokenize(E, Wp, bp))
    ref = oracle.tokenize(ti.E, ti.Wp, ti.bp)
    _check(X, ref, dtype, f"tokenize {B}x{T}x{d}->{D} {dtype}")


def test_tokenize_without_bias_and_reuse_of_output():
    import torch
    import rankmixer_block_forward_amd as rmx
    ti = synth.make_tokenize_inputs(40, 3, 64, 128, "bf16", seed=3)
    E, Wp, _ = _upload(ti, "bf16")
    X = torch.full((40, 3, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    rmx.tokenize(E, Wp, None, X=X)
    _check(to_np(X), oracle.tokenize(ti.E, ti.Wp, np.zeros((3, 128))), "bf16", "tokenize no bias")


def test_tokenize_1b_input_full_size():
    """The 1B shape's input: B = 2048, T = 32, d = 512 -> D = 1536, checked on sampled rows."""
    import rankmixer_block_forward_amd as rmx
    B, T, d, D = 2048, 32, synth.TOKENIZE_D, 1536
    ti = synth.make_tokenize_inputs(B, T, d, D, "bf16", seed=0)
    E, Wp, bp = _upload(ti, "bf16")
    X = to_np(rmx.tokenize(E, Wp, bp))
    rows = sample_rows(B, 16)
    _check(X[rows], oracle.tokenize(ti.E[rows], ti.Wp, ti.bp), "bf16", "tokenize 1B input")


def test_tokenize_then_block_forward_matches_oracle_pipeline():
    """The tokens the projection writes feed rmx_block_forward directly."""
    import torch
    import rankmixer_block_forward_amd as rmx
    cfg = synth.Config("tok", B=24, T=4, D=128, k=2, L=2, dtype="bf16", bias_std=0.02)
    inp = synth.make_inputs(cfg, seed=5)
    ti = synth.make_tokenize_inputs(cfg.B, cfg.T, 64, cfg.D, "bf16", seed=5, bias_std=0.02)
    E, Wp, bp = _upload(ti, "bf16")
    X = rmx.tokenize(E, Wp, bp)
    _, w = rmx.upload(inp)
    with rmx.Handle.for_config(cfg, max_batch=cfg.B) as h:
        out = h.forward(X, w)
        torch.cuda.synchronize()
    Xg = to_np(X).astype(np.float64)           # the tokens as the GPU rounded them
    o_ref, _, _ = oracle.forward(Xg, inp.layers(), cfg.eps)
    _check(to_np(out), o_ref, "bf16", "tokenize -> forward")
    _check(Xg, oracle.tokenize(ti.E, ti.Wp, ti.bp), "bf16", "tokens")


def test_tokenize_errors_and_empty_batch():
    import torch
    import rankmixer_block_forward_amd as rmx
    from rankmixer_block_forward_amd import binding
    ti = synth.make_tokenize_inputs(8, 2, 32, 64, "bf16", seed=1)
    E, Wp, bp = _upload(ti, "bf16")
    X = torch.full((8, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    lib = binding.load_library()
    # E too small for the stated batch: rejected on the host, X untouched
    st = lib.rmx_tokenize(E.data_ptr(), Wp.data_ptr(), bp.data_ptr(), X.data_ptr(), 1 << 20, 2, 32, 64, 1, None)
    assert st == binding.RMX_ERR_INVALID_ARG and "E" in lib.rmx_last_error(None).decode()
    # overlapping input and output
    st = lib.rmx_tokenize(E.data_ptr(), Wp.data_ptr(), bp.data_ptr(), E.data_ptr(), 8, 2, 32, 32, 1, None)
    assert st == binding.RMX_ERR_INVALID_ARG
    st = lib.rmx_tokenize(E.data_ptr(), Wp.data_ptr(), bp.data_ptr(), X.data_ptr(), 0, 2, 32, 64, 1, None)
    assert st == binding.RMX_OK
    torch.cuda.synchronize()
    assert torch.all(X == 7.0)
