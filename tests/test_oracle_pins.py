"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or the mathematics fix:
values the pages print (tests/golden/, each file carries its citation), closed forms,
invariants, special cases that reduce to a library routine (torch.nn.functional in
fp64, scipy.stats), and a scalar-loop brute force on tiny shapes.  Together they are
chosen so that a dropped term, a wrong sign, axis or index, or a transposed operand in
the oracle fails at least one of them.
"""
import numpy as np
import pytest
import scipy.stats
import torch
import torch.nn.functional as F

import oracle
from oracle import brute
from rankmixer_block_forward_amd import synth
from tests.golden_io import read

EPS = 1e-5


# --------------------------------------------------------------------------- mixing

def test_mix_labelled_4_tokens_8_dims():
    """Mixed token h = head h of tokens A, B, C, D in token order (4 x 8 example)."""
    g = read("mix_4tokens_8dims.txt", labels=True)
    T, H, q = 4, 4, 2
    labels = g["input"]
    # encode head label (token t, head h) and coordinate r as a unique number
    code = {labels[t][h]: 1000 * (t + 1) + 10 * (h + 1) for t in range(T) for h in range(H)}
    X = np.zeros((T, H * q))
    for t in range(T):
        for h in range(H):
            X[t, h * q:(h + 1) * q] = [code[labels[t][h]] + r for r in range(q)]
    M = oracle.token_mix(X)
    for h in range(T):
        for s in range(T):
            want = [code[g["output"][h][s]] + r for r in range(q)]
            assert list(M[h, s * q:(s + 1) * q]) == want


def test_mix_unimixer_appendix_example_and_permutation_matrix():
    g = read("unimixer_appendix_a.txt")
    X = g["X"]
    assert np.array_equal(oracle.token_mix(X), g["mixed"])
    # The permutation matrix of the oracle's map, column by column from basis vectors.
    n = X.size
    P = np.zeros((n, n))
    for i in range(n):
        e = np.zeros(n)
        e[i] = 1.0
        P[:, i] = oracle.token_mix(e.reshape(X.shape)).reshape(-1)
    assert np.array_equal(P, g["W_perm"])
    assert np.array_equal(P, np.kron(g["G"], np.eye(3)))
    # permutation properties stated with the example: doubly stochastic, one nonzero
    # per row/column, symmetric when T = H
    assert np.array_equal(P.sum(0), np.ones(n)) and np.array_equal(P.sum(1), np.ones(n))
    assert np.array_equal(P, P.T)


@pytest.mark.parametrize("T,D", [(2, 6), (4, 8), (4, 4), (3, 12), (8, 64), (16, 768)])
def test_mix_is_symmetric_permutation(T, D):
    rng = np.random.default_rng(T * 1000 + D)
    X = rng.standard_normal((5, T, D))
    M = oracle.token_mix(X)
    # involution: the permutation equals its transpose, so applying it twice is identity
    assert np.array_equal(oracle.token_mix(M), X)
    # a permutation within each sample: the multiset of values is preserved
    assert np.array_equal(np.sort(M.reshape(5, -1), 1), np.sort(X.reshape(5, -1), 1))
    # the array form: view X as T x H x q, swap the first two axes, merge the last two
    q = D // T
    Mr = X.reshape(5, T, T, q).transpose(0, 2, 1, 3).reshape(5, T, D)
    assert np.array_equal(M, Mr)


def test_mix_is_transpose_when_heads_have_one_coordinate():
    X = np.arange(16.0).reshape(4, 4)
    assert np.array_equal(oracle.token_mix(X), X.T)


def test_mix_rejects_indivisible_width():
    with pytest.raises(ValueError):
        oracle.token_mix(np.zeros((3, 8)))


# ---------------------------------------------------------------- worked example

def test_worked_example_mixing_plus_residual():
    g = read("rankmixer_worked_example.txt")
    R = oracle.token_mix(g["X0"]) + g["X0"]
    # inputs carry 4-decimal rounding; the sum of two rounded values is within 1e-4
    np.testing.assert_allclose(R, g["R"], atol=1.01e-4, rtol=0)


def test_worked_example_first_layernorm():
    g = read("rankmixer_worked_example.txt")
    R = g["R"]
    r0 = R[0]
    assert abs(r0.mean() - g["row1_mean"][0, 0]) < 1e-4
    assert abs(((r0 - r0.mean()) ** 2).mean() - g["row1_var"][0, 0]) < 1e-4
    S0 = oracle.layer_norm(R, np.ones(4), np.zeros(4), EPS)
    assert abs(S0[0, 0] - g["S0_first"][0, 0]) < 1e-4
    np.testing.assert_allclose(S0, g["S0"], atol=3e-4, rtol=0)
    # the printed values separate the biased variance from the D-1 one
    unbiased = (R - R.mean(1, keepdims=True)) / np.sqrt(R.var(1, ddof=1, keepdims=True) + EPS)
    assert np.abs(unbiased - g["S0"]).max() > 0.05


def test_worked_example_second_layernorm_and_pool():
    g = read("rankmixer_worked_example.txt")
    X1 = oracle.layer_norm(g["S0"] + g["V"], np.ones(4), np.zeros(4), EPS)
    np.testing.assert_allclose(X1, g["X1"], atol=3e-4, rtol=0)
    # the pool: forward() with no blocks returns the mean over tokens of its input
    o, XL, _ = oracle.forward(g["X1"][None], [], EPS)
    np.testing.assert_allclose(o[0], g["o"][0], atol=1.01e-4, rtol=0)
    assert np.array_equal(XL[0], g["X1"])


def test_worked_example_gelu_of_u1():
    g = read("rankmixer_worked_example.txt")
    a = oracle.gelu(g["u1"][0])
    assert abs(a[0] - g["gelu_u1_first"][0, 0]) < 1e-4
    assert abs(a[3] - g["gelu_u1_fourth"][0, 0]) < 1e-4


# ------------------------------------------------------------------------ GELU

def test_gelu_printed_values():
    g = read("gelu_values.txt")
    assert abs(oracle.gelu(1.0) - g["gelu_plus1"][0, 0]) < 5e-5
    assert abs(oracle.gelu(-1.0) - g["gelu_minus1"][0, 0]) < 5e-5
    C = oracle.gelu(2.0) - 2 * oracle.gelu(1.0) + oracle.gelu(0.0)
    assert abs(C - g["interaction_C"][0, 0]) < 5e-5
    # the printed C rules out the tanh approximation (it gives 0.2722)
    tanh = lambda u: 0.5 * u * (1 + np.tanh(np.sqrt(2 / np.pi) * (u + 0.044715 * u ** 3)))
    assert abs(tanh(2.0) - 2 * tanh(1.0) - g["interaction_C"][0, 0]) > 2e-4


def test_gelu_is_u_times_normal_cdf():
    u = np.linspace(-8, 8, 2001)
    np.testing.assert_allclose(oracle.gelu(u), u * scipy.stats.norm.cdf(u), rtol=1e-13, atol=1e-15)
    t = torch.tensor(u, dtype=torch.float64)
    np.testing.assert_allclose(oracle.gelu(u), F.gelu(t, approximate="none").numpy(), rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------- LayerNorm

def test_layernorm_matches_torch_and_row_moments():
    rng = np.random.default_rng(1)
    R = rng.standard_normal((7, 5, 33)) * 3 + 2
    g, b = rng.standard_normal(33), rng.standard_normal(33)
    out = oracle.layer_norm(R, g, b, EPS)
    ref = F.layer_norm(torch.tensor(R), (33,), torch.tensor(g), torch.tensor(b), EPS).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # with gamma = 1, beta = 0: every row has mean 0 and variance var / (var + eps)
    n = oracle.layer_norm(R, np.ones(33), np.zeros(33), EPS)
    var = R.var(-1)
    np.testing.assert_allclose(n.mean(-1), 0, atol=1e-13)
    np.testing.assert_allclose(n.var(-1), var / (var + EPS), rtol=1e-12)


def test_layernorm_shift_invariance_and_page_example():
    # [1,2,3,4] and [11,12,13,14] centre to the same vector, so normalise identically
    a = oracle.layer_norm(np.array([[1.0, 2, 3, 4], [11, 12, 13, 14]]), np.ones(4), np.zeros(4), EPS)
    assert np.allclose(a[0], a[1], atol=1e-12)
    np.testing.assert_allclose(a[0], np.array([-1.5, -0.5, 0.5, 1.5]) / np.sqrt(1.25 + EPS), rtol=1e-13)


def test_layernorm_zero_row_gives_beta():
    b = np.arange(6.0)
    out = oracle.layer_norm(np.zeros((2, 6)), np.full(6, 3.0), b, EPS)
    assert np.array_equal(out, np.stack([b, b]))


# ------------------------------------------------------------------------ PFFN

def _rand_ffn(rng, T, D, k, bias=0.1):
    W1 = rng.standard_normal((T, D, k * D)) / np.sqrt(D)
    W2 = rng.standard_normal((T, k * D, D)) / np.sqrt(k * D)
    return W1, bias * rng.standard_normal((T, k * D)), W2, bias * rng.standard_normal((T, D))


def _torch_mlp(x, W1, b1, W2, b2):
    """Textbook 2-layer MLP with torch's Linear convention (weight is out x in)."""
    x = torch.tensor(x)
    h = F.gelu(F.linear(x, torch.tensor(W1).T, torch.tensor(b1)), approximate="none")
    return F.linear(h, torch.tensor(W2).T, torch.tensor(b2)).numpy()


def test_pffn_with_equal_weights_is_one_shared_mlp():
    rng = np.random.default_rng(2)
    T, D, k = 5, 12, 3
    W1, b1, W2, b2 = _rand_ffn(rng, 1, D, k)
    S = rng.standard_normal((6, T, D))
    V = oracle.pffn(S, np.repeat(W1, T, 0), np.repeat(b1, T, 0), np.repeat(W2, T, 0), np.repeat(b2, T, 0))
    ref = _torch_mlp(S.reshape(-1, D), W1[0], b1[0], W2[0], b2[0]).reshape(6, T, D)
    np.testing.assert_allclose(V, ref, rtol=1e-12, atol=1e-12)


def test_pffn_is_block_diagonal_mlp_over_flattened_tokens():
    """Per-token weights = one MLP on the flattened [T*D] row with block-diagonal weights."""
    rng = np.random.default_rng(3)
    T, D, k = 4, 6, 2
    W1, b1, W2, b2 = _rand_ffn(rng, T, D, k)
    S = rng.standard_normal((9, T, D))
    V = oracle.pffn(S, W1, b1, W2, b2)
    bd1 = torch.block_diag(*[torch.tensor(w) for w in W1]).numpy()
    bd2 = torch.block_diag(*[torch.tensor(w) for w in W2]).numpy()
    ref = _torch_mlp(S.reshape(9, T * D), bd1, b1.reshape(-1), bd2, b2.reshape(-1)).reshape(9, T, D)
    np.testing.assert_allclose(V, ref, rtol=1e-12, atol=1e-12)


def test_pffn_token_permutation_equivariance():
    rng = np.random.default_rng(4)
    T, D, k = 6, 6, 2
    W1, b1, W2, b2 = _rand_ffn(rng, T, D, k)
    S = rng.standard_normal((3, T, D))
    perm = rng.permutation(T)
    V = oracle.pffn(S, W1, b1, W2, b2)
    Vp = oracle.pffn(S[:, perm], W1[perm], b1[perm], W2[perm], b2[perm])
    np.testing.assert_allclose(Vp, V[:, perm], rtol=1e-13, atol=1e-13)


# -------------------------------------------------------------- whole forward

def _params(rng, T, D, k, L, moe_E=0, h=0):
    layers = []
    for _ in range(L):
        W1, b1, W2, b2 = _rand_ffn(rng, T, D, k)
        p = dict(W1=W1, b1=b1, W2=W2, b2=b2,
                 ln1_g=1 + 0.3 * rng.standard_normal(D), ln1_b=0.3 * rng.standard_normal(D),
                 ln2_g=1 + 0.3 * rng.standard_normal(D), ln2_b=0.3 * rng.standard_normal(D))
        if moe_E:
            p.update(Wg=rng.standard_normal((T, D, moe_E)) / np.sqrt(D),
                     We1=rng.standard_normal((T, moe_E, D, h)) / np.sqrt(D),
                     be1=0.1 * rng.standard_normal((T, moe_E, h)),
                     We2=rng.standard_normal((T, moe_E, h, D)) / np.sqrt(h),
                     be2=0.1 * rng.standard_normal((T, moe_E, D)))
        layers.append(p)
    return layers


@pytest.mark.parametrize("T,D,k,L", [(4, 8, 2, 1), (2, 6, 2, 2), (3, 9, 1, 2), (4, 4, 3, 1)])
def test_forward_matches_scalar_brute_force(T, D, k, L):
    rng = np.random.default_rng(T * 100 + D * 10 + L)
    X = rng.standard_normal((3, T, D))
    layers = _params(rng, T, D, k, L)
    o, XL, _ = oracle.forward(X, layers, EPS)
    for b in range(3):
        ob, xb, _ = brute.forward_sample(X[b], layers, EPS)
        np.testing.assert_allclose(o[b], ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(XL[b], xb, rtol=1e-12, atol=1e-12)


def test_forward_tiny_workload_matches_brute_force():
    inp = synth.make_inputs(synth.TINY, seed=0)
    o, XL, _ = oracle.forward(inp.X, inp.layers(), EPS)
    assert o.shape == (8, 8) and XL.shape == (8, 4, 8)
    for b in range(8):
        ob, xb, _ = brute.forward_sample(inp.X[b], inp.layers(), EPS)
        np.testing.assert_allclose(o[b], ob, rtol=1e-12, atol=1e-12)
    # every row of X_L is a LayerNorm output with gamma = 1, beta = 0
    np.testing.assert_allclose(XL.mean(-1), 0, atol=1e-12)
    np.testing.assert_allclose(XL.var(-1), 1, atol=1e-3)


def test_forward_tiny_golden():
    """Regression pin: the tiny workload's output, written by tests/golden/make_golden.py."""
    g = read("tiny_oracle_output.txt")
    inp = synth.make_inputs(synth.TINY, seed=0)
    o, _, _ = oracle.forward(inp.X, inp.layers(), EPS)
    np.testing.assert_allclose(o, g["o"], rtol=0, atol=1e-12)


def test_zero_token_rows_stay_finite():
    cfg = synth.TINY.with_(zero_frac=0.5, B=4)
    inp = synth.make_inputs(cfg, seed=0)
    assert (np.abs(inp.X).sum(-1) == 0).sum() == 8
    o, XL, _ = oracle.forward(inp.X, inp.layers(), EPS)
    assert np.isfinite(o).all() and np.isfinite(XL).all()


# ----------------------------------------------------------------- Sparse-MoE

def test_moe_matches_scalar_brute_force():
    rng = np.random.default_rng(11)
    T, D, k, E, h = 3, 6, 2, 4, 5
    X = rng.standard_normal((4, T, D))
    layers = _params(rng, T, D, k, 2, moe_E=E, h=h)
    o, XL, gates = oracle.forward(X, layers, EPS)
    assert all(G is not None and G.shape == (4, T, E) for G in gates)
    assert (gates[0] == 0).any() and (gates[0] > 0).any()
    for b in range(4):
        ob, xb, gb = brute.forward_sample(X[b], layers, EPS)
        np.testing.assert_allclose(o[b], ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(gates[0][b], np.array(gb[0]), rtol=1e-12, atol=1e-12)


def test_moe_zero_router_gives_layernorm_of_s():
    rng = np.random.default_rng(12)
    T, D, E, h = 4, 8, 3, 6
    p = _params(rng, T, D, 2, 1, moe_E=E, h=h)[0]
    p["Wg"] = np.zeros_like(p["Wg"])
    X = rng.standard_normal((5, T, D))
    Xn, G = oracle.block(X, p, EPS)
    assert not G.any()
    S = oracle.layer_norm(oracle.token_mix(X) + X, p["ln1_g"], p["ln1_b"], EPS)
    np.testing.assert_allclose(Xn, oracle.layer_norm(S, p["ln2_g"], p["ln2_b"], EPS), rtol=1e-13, atol=1e-13)


def test_moe_router_positive_homogeneity():
    rng = np.random.default_rng(13)
    T, D, E, h = 3, 6, 4, 5
    p = _params(rng, T, D, 2, 1, moe_E=E, h=h)[0]
    S = rng.standard_normal((6, T, D))
    V1, G1 = oracle.moe_pffn(S, p["Wg"], p["We1"], p["be1"], p["We2"], p["be2"])
    V3, G3 = oracle.moe_pffn(S, 3.0 * p["Wg"], p["We1"], p["be1"], p["We2"], p["be2"])
    np.testing.assert_allclose(G3, 3.0 * G1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(V3, 3.0 * V1, rtol=1e-12, atol=1e-13)


def test_moe_equal_experts_scale_one_mlp():
    rng = np.random.default_rng(14)
    T, D, E, h = 3, 6, 4, 5
    p = _params(rng, T, D, 2, 1, moe_E=E, h=h)[0]
    for name in ("We1", "be1", "We2", "be2"):
        p[name] = np.repeat(p[name][:, :1], E, axis=1)
    S = rng.standard_normal((7, T, D))
    V, G = oracle.moe_pffn(S, p["Wg"], p["We1"], p["be1"], p["We2"], p["be2"])
    for t in range(T):
        y = _torch_mlp(S[:, t], p["We1"][t, 0], p["be1"][t, 0], p["We2"][t, 0], p["be2"][t, 0])
        np.testing.assert_allclose(V[:, t], G[:, t].sum(-1)[:, None] * y, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------- tokenisation

def test_tokenize_identity_projection_takes_half_open_slices():
    """d = D, Wp[t] = I, bp = 0: token t is exactly coordinates t*d .. t*d + d - 1 of the
    concatenated embedding, the first d going to the first token ([exp1] 2: half-open
    slices, first slice the first d coordinates)."""
    T, d, B = 3, 4, 2
    E = np.arange(B * T * d, dtype=np.float64).reshape(B, T * d)
    X = oracle.tokenize(E, np.stack([np.eye(d)] * T), np.zeros((T, d)))
    assert X.shape == (B, T, d)
    assert X[0, 0].tolist() == [0.0, 1.0, 2.0, 3.0]
    assert X[0, 2].tolist() == [8.0, 9.0, 10.0, 11.0]
    assert X[1, 1].tolist() == [16.0, 17.0, 18.0, 19.0]


def test_tokenize_shared_weights_is_one_linear_layer():
    """All tokens given the same layer: one torch Linear over the [B, T, d] view."""
    rng = np.random.default_rng(11)
    T, d, D, B = 4, 5, 7, 6
    W = rng.standard_normal((d, D))
    b = rng.standard_normal(D)
    E = rng.standard_normal((B, T * d))
    X = oracle.tokenize(E, np.stack([W] * T), np.stack([b] * T))
    ref = F.linear(torch.tensor(E).view(B, T, d), torch.tensor(W).T, torch.tensor(b)).numpy()
    np.testing.assert_allclose(X, ref, rtol=1e-12, atol=1e-12)


def test_tokenize_token_specific_is_block_diagonal_linear():
    """Token-specific layers ([uni] eq (9)) = one Linear over the whole embedding with a
    block-diagonal weight whose t-th block is Wp[t]."""
    rng = np.random.default_rng(12)
    T, d, D, B = 3, 4, 6, 5
    Wp = rng.standard_normal((T, d, D))
    bp = rng.standard_normal((T, D))
    E = rng.standard_normal((B, T * d))
    X = oracle.tokenize(E, Wp, bp)
    bd = torch.block_diag(*[torch.tensor(w) for w in Wp])            # [T*d, T*D]
    ref = F.linear(torch.tensor(E), bd.T, torch.tensor(bp.reshape(-1))).numpy().reshape(B, T, D)
    np.testing.assert_allclose(X, ref, rtol=1e-12, atol=1e-12)


def test_tokenize_matches_scalar_brute_force():
    rng = np.random.default_rng(13)
    T, d, D, B = 3, 5, 4, 4
    Wp = rng.standard_normal((T, d, D))
    bp = rng.standard_normal((T, D))
    E = rng.standard_normal((B, T * d))
    X = oracle.tokenize(E, Wp, bp)
    for b in range(B):
        np.testing.assert_allclose(X[b], np.array(brute.tokenize_sample(E[b], Wp, bp)), rtol=1e-13, atol=1e-13)


def test_tokenize_rejects_wrong_width():
    with pytest.raises(ValueError):
        oracle.tokenize(np.zeros((2, 7)), np.zeros((2, 4, 3)), np.zeros((2, 3)))
