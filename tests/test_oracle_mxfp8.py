"""Pins of the MXFP8 oracle (CPU only).

The quantizer follows the OCP Microscaling Formats (MX) Specification v1.0 for MXFP8 with
E4M3 elements.  Pinned by: the library's FP8 E4M3 cast (torch.float8_e4m3fn, after
saturation at +-448) on values across every binade and on exact rounding ties; the E4M3
grid itself (every finite code decodes to a fixed point of the rounding); closed forms of
the shared exponent; invariances of block quantization; a worked block; and a scalar
brute-force twin of the quantized forward on tiny shapes (catches a wrong quantization axis).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import rmx_mxfp8 as mx

EPS = 1e-5


def _torch_e4m3(v):
    t = torch.tensor(np.clip(v, -448.0, 448.0), dtype=torch.float64).to(torch.float32)
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_rounding_matches_the_library_cast():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-14, 10, 20000))
    np.testing.assert_array_equal(oracle.e4m3_round(v), _torch_e4m3(v))


def test_e4m3_rounding_ties_go_to_even_and_saturate():
    grid = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = np.unique(grid[np.isfinite(grid)])
    assert finite.max() == 448.0 and finite[finite > 0].min() == 2.0 ** -9
    np.testing.assert_array_equal(oracle.e4m3_round(finite), finite)   # the grid is fixed
    pos = finite[finite >= 0]
    mids = (pos[:-1] + pos[1:]) / 2                                     # exact ties
    np.testing.assert_array_equal(oracle.e4m3_round(mids), _torch_e4m3(mids))
    assert oracle.e4m3_round(1.0625) == 1.0 and oracle.e4m3_round(1.1875) == 1.25
    assert oracle.e4m3_round(1e9) == 448.0 and oracle.e4m3_round(-500.0) == -448.0
    assert oracle.e4m3_round(2.0 ** -10) == 0.0 and oracle.e4m3_round(1.5 * 2.0 ** -10) == 2.0 ** -9


def test_shared_exponent_closed_forms():
    e = oracle.mx_scale_exponent
    assert e(1.0) == -8 and e(448.0) == 0 and e(256.0) == 0 and e(255.9) == -1
    assert e(2.0 ** 20) == 12 and e(0.0) == -127
    assert e(2.0 ** 200) == 127 and e(2.0 ** -200) == -127
    for k in range(-20, 20):
        assert e(2.0 ** k) == k - 8 and e(np.nextafter(2.0 ** k, 0)) == k - 9


def test_block_max_lands_in_the_top_binade():
    """After scaling, a block's largest magnitude lies in [256, 512) and is stored as a
    value in [256, 448]."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 32)) * np.exp2(rng.integers(-30, 30, (50, 1)))
    q = oracle.mx_qdq(x)
    e = oracle.mx_scale_exponent(np.abs(x).max(-1))
    top = np.abs(q).max(-1) / np.exp2(e)
    assert np.all((top >= 256) & (top <= 448))


def test_block_quantization_invariances():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 96))
    q = oracle.mx_qdq(x)
    np.testing.assert_array_equal(oracle.mx_qdq(q), q)                 # idempotent
    for k in (-7, 3, 11):                                               # power-of-two scaling
        np.testing.assert_array_equal(oracle.mx_qdq(np.ldexp(x, k)), np.ldexp(q, k))
    y = x.copy()
    y[:, 32:64] *= 1000.0                                               # blocks are independent
    qy = oracle.mx_qdq(y)
    np.testing.assert_array_equal(qy[:, :32], q[:, :32])
    np.testing.assert_array_equal(qy[:, 64:], q[:, 64:])
    np.testing.assert_array_equal(oracle.mx_qdq(x.T, axis=0), q.T)     # the axis argument
    scale = np.exp2(oracle.mx_scale_exponent(np.abs(x).reshape(6, 3, 32).max(-1))).repeat(32, 1)
    rel = np.abs(q - x) / np.abs(x)
    normal = (np.abs(x) >= scale * 2.0 ** -6) & (np.abs(x) <= scale * 448)
    assert rel[normal].max() <= 2.0 ** -4                               # half an E4M3 ulp
    # a block maximum scaled into (448, 512) saturates at 448: at most 1/8 relative
    assert rel[np.abs(x) > scale * 448].max(initial=0.0) <= 0.125
    with pytest.raises(ValueError):
        oracle.mx_qdq(np.ones((2, 40)))


def test_worked_block():
    """Block 1..32: amax 32 gives X = 2^(5-8) = 1/8; v = 8 k.  Up to 128 (k <= 16) every v is
    on the grid; from 128 to 256 the step is 16, so 8 k rounds to an even multiple of 16
    when it falls half way: k = 17 (136) -> 128, k = 19 (152) -> 160, k = 18 -> 144."""
    q = oracle.mx_qdq(np.arange(1, 33, dtype=np.float64))
    np.testing.assert_array_equal(q[:16], np.arange(1, 17))
    assert q[16] == 16.0 and q[17] == 18.0 and q[18] == 20.0 and q[31] == 32.0


# ---------------------------------------------------------- quantized forward

def _q_scalar(vals):
    """MX quantize-dequantize of one 32-value block with Python floats."""
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        return [0.0] * len(vals)
    e = math.frexp(amax)[1] - 1 - 8
    out = []
    for v in vals:
        s = v / 2.0 ** e
        a = abs(s)
        E = max(math.frexp(a)[1] - 1 if a > 0 else -6, -6)
        qnt = 2.0 ** (E - 3)
        r = round(s / qnt) * qnt                       # Python round: ties to even
        out.append(max(-448.0, min(448.0, r)) * 2.0 ** e)
    return out


def _brute_forward_mxfp8(X, layers, eps):
    """Scalar twin of forward_mxfp8 for shapes with D = k D = 32 (one block per row / column)."""
    from oracle import brute
    X = [[list(map(float, row)) for row in sample] for sample in np.asarray(X)]
    out = []
    for x in X:
        for p in layers:
            T, D = len(x), len(x[0])
            m = brute._mix(x, T, D)
            S = [brute._ln_row([m[h][c] + x[h][c] for c in range(D)], p["ln1_g"], p["ln1_b"], eps) for h in range(T)]
            Y = []
            for t in range(T):
                s = _q_scalar(S[t])
                W1, W2 = np.asarray(p["W1"][t]), np.asarray(p["W2"][t])
                kD = W1.shape[1]
                w1 = [_q_scalar([W1[d][j] for d in range(D)]) for j in range(kD)]     # column j along K
                u = [sum(s[d] * w1[j][d] for d in range(D)) + p["b1"][t][j] for j in range(kD)]
                hq = _q_scalar([brute._gelu(v) for v in u])
                w2 = [_q_scalar([W2[j][c] for j in range(kD)]) for c in range(D)]
                v = [sum(hq[j] * w2[c][j] for j in range(kD)) + p["b2"][t][c] for c in range(D)]
                Y.append(brute._ln_row([v[c] + S[t][c] for c in range(D)], p["ln2_g"], p["ln2_b"], eps))
            x = Y
        out.append(x)
    return np.array(out)


def test_forward_mxfp8_matches_scalar_twin():
    rng = np.random.default_rng(3)
    B, T, D, k, L = 2, 2, 32, 1, 2
    X = rng.standard_normal((B, T, D))
    layers = []
    for _ in range(L):
        layers.append(dict(W1=rng.standard_normal((T, D, k * D)) / np.sqrt(D),
                           b1=0.1 * rng.standard_normal((T, k * D)),
                           W2=rng.standard_normal((T, k * D, D)) / np.sqrt(k * D),
                           b2=0.1 * rng.standard_normal((T, D)),
                           ln1_g=1 + 0.2 * rng.standard_normal(D), ln1_b=0.2 * rng.standard_normal(D),
                           ln2_g=1 + 0.2 * rng.standard_normal(D), ln2_b=0.2 * rng.standard_normal(D)))
    o, XL = oracle.forward_mxfp8(X, layers, EPS)
    ref = _brute_forward_mxfp8(X, layers, EPS)
    np.testing.assert_allclose(XL, ref, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(o, ref.mean(1), rtol=1e-9, atol=1e-9)
    # quantization moves the result, but only at the format's precision
    o_ref, XL_ref, _ = oracle.forward(X, layers, EPS)
    err = np.linalg.norm(XL - XL_ref) / np.linalg.norm(XL_ref)
    assert 1e-4 < err < 0.2


def test_forward_mxfp8_is_forward_when_every_operand_is_representable():
    """With the quantizer replaced by the identity, the quantized forward is the forward."""
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3, 4, 32))
    p = dict(W1=rng.standard_normal((4, 32, 64)) / 6, b1=0.1 * rng.standard_normal((4, 64)),
             W2=rng.standard_normal((4, 64, 32)) / 8, b2=0.1 * rng.standard_normal((4, 32)),
             ln1_g=np.ones(32), ln1_b=np.zeros(32), ln2_g=np.ones(32), ln2_b=np.zeros(32))
    saved = mx.mx_qdq
    try:
        mx.mx_qdq = lambda x, axis=-1: np.asarray(x, dtype=np.float64)
        o, XL = oracle.forward_mxfp8(X, [p], EPS)
    finally:
        mx.mx_qdq = saved
    o_ref, XL_ref, _ = oracle.forward(X, [p], EPS)
    np.testing.assert_allclose(XL, XL_ref, rtol=1e-13, atol=1e-13)


def test_prequantized_weights_give_the_same_bits():
    """forward_mxfp8 with the weights quantized beforehand (on threads) returns exactly what
    it returns when it quantizes them itself: the same function of the same values."""
    from rankmixer_block_forward_amd import synth
    cfg = synth.Config("mx-pre", B=6, T=4, D=64, k=2, L=2, bias_std=0.05)
    inp = synth.make_inputs(cfg, seed=4)
    a = oracle.forward_mxfp8(inp.X, inp.layers(), EPS)
    wq = oracle.quantize_weights(inp.layers(), workers=4)
    b = oracle.forward_mxfp8(inp.X, inp.layers(), EPS, wq=wq)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    assert np.array_equal(wq[1][3][0], oracle.mx_qdq(inp.layers()[1]["W1"][3], axis=0))
