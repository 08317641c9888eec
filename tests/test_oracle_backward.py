"""Pins of the fp64 backward oracle (CPU only).

The backward oracle follows the gradients written out in "RankMixer 详解（1）：特征分组与
完整计算流程" (jackknifer.me), section 5.2.  None of the page's intermediate gradients of
the block are printed (its FFN weights are not), so the oracle is pinned by what fixes a
gradient independently of how it is written down:
  * central finite differences of the forward oracle (itself pinned to the pages' worked
    example, closed forms and brute force in test_oracle_pins.py), on every coordinate of a
    small stack and on sampled coordinates of larger ones;
  * the adjoint identity <P x, g> = <x, P^T g> of the mixing permutation, and P^T = P;
  * a library autograd of a textbook two-layer MLP (shared weights, and per-token weights as
    one block-diagonal MLP);
  * closed forms and limits of GELU' and the shift invariance of LayerNorm;
  * the page's worked prediction-head numbers (section 6.4), fixture
    tests/golden/prediction_head_example.txt.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests.golden_io import read

EPS = 1e-5


def _params(rng, T, D, k, L, bias=0.3):
    layers = []
    for _ in range(L):
        layers.append(dict(
            W1=rng.standard_normal((T, D, k * D)) / np.sqrt(D),
            b1=bias * rng.standard_normal((T, k * D)),
            W2=rng.standard_normal((T, k * D, D)) / np.sqrt(k * D),
            b2=bias * rng.standard_normal((T, D)),
            ln1_g=1 + 0.3 * rng.standard_normal(D), ln1_b=0.3 * rng.standard_normal(D),
            ln2_g=1 + 0.3 * rng.standard_normal(D), ln2_b=0.3 * rng.standard_normal(D)))
    return layers


def _loss(X, layers, g_o):
    o, _, _ = oracle.forward(X, layers, EPS)
    return float((o * g_o).sum())


def _fd(f, arr, idx, h=1e-5):
    """Central difference of f() in arr[idx] (arr is perturbed in place and restored)."""
    old = arr[idx]
    arr[idx] = old + h
    fp = f()
    arr[idx] = old - h
    fm = f()
    arr[idx] = old
    return (fp - fm) / (2 * h)


def _check_fd(X, layers, g_o, coords_per_tensor=None, seed=0):
    """Compare the oracle's gradients with central differences of sum(g_o * o)."""
    dX, grads = oracle.backward(X, layers, g_o, EPS)
    f = lambda: _loss(X, layers, g_o)  # noqa: E731
    rng = np.random.default_rng(seed)
    tensors = [("X", X, dX)] + [(f"{name}[{n}]", layers[n][name], grads[n][name])
                                for n in range(len(layers)) for name in layers[n]]
    for label, arr, grad in tensors:
        assert grad.shape == arr.shape, label
        if coords_per_tensor is None:
            idxs = list(np.ndindex(arr.shape))
        else:
            flat = rng.choice(arr.size, size=min(coords_per_tensor, arr.size), replace=False)
            idxs = [np.unravel_index(i, arr.shape) for i in flat]
        for idx in idxs:
            num = _fd(f, arr, idx)
            assert abs(num - grad[idx]) <= 1e-7 * max(1.0, abs(num)), (label, idx, num, grad[idx])


# ------------------------------------------------------------- finite differences

def test_backward_every_coordinate_matches_central_differences():
    """T = 2, D = 4, k = 2, L = 2: every coordinate of X and of every parameter."""
    rng = np.random.default_rng(11)
    B, T, D, k, L = 2, 2, 4, 2, 2
    X = rng.standard_normal((B, T, D))
    layers = _params(rng, T, D, k, L)
    g_o = rng.standard_normal((B, D))
    _check_fd(X, layers, g_o)


@pytest.mark.parametrize("B,T,D,k,L", [(3, 4, 8, 2, 2), (2, 3, 9, 1, 1), (2, 4, 12, 3, 2)])
def test_backward_sampled_coordinates_match_central_differences(B, T, D, k, L):
    rng = np.random.default_rng(100 * T + D + L)
    X = rng.standard_normal((B, T, D))
    layers = _params(rng, T, D, k, L)
    g_o = rng.standard_normal((B, D))
    _check_fd(X, layers, g_o, coords_per_tensor=6, seed=T + D)


def test_backward_with_zero_token_row_matches_central_differences():
    """A zero input row (the sweep's zeroed tokens) stays differentiable: eps keeps the
    LayerNorm's rstd finite."""
    rng = np.random.default_rng(12)
    X = rng.standard_normal((2, 4, 8))
    X[1, 2] = 0.0
    layers = _params(rng, 4, 8, 2, 1)
    g_o = rng.standard_normal((2, 8))
    _check_fd(X, layers, g_o, coords_per_tensor=8)


def test_pool_sends_each_row_g_over_T():
    """With no blocks, o = mean_t X[:, t]: every row receives g_o / T ([exp1] 5.2)."""
    rng = np.random.default_rng(13)
    g_o = rng.standard_normal((3, 6))
    dX, grads = oracle.backward(rng.standard_normal((3, 5, 6)), [], g_o, EPS)
    assert grads == []
    np.testing.assert_array_equal(dX, np.broadcast_to(g_o[:, None, :] / 5, (3, 5, 6)))


def test_backward_is_linear_in_the_upstream_gradient():
    rng = np.random.default_rng(14)
    X = rng.standard_normal((2, 4, 8))
    layers = _params(rng, 4, 8, 2, 2)
    g1, g2 = rng.standard_normal((2, 2, 8))
    d1, p1 = oracle.backward(X, layers, g1, EPS)
    d2, p2 = oracle.backward(X, layers, g2, EPS)
    d3, p3 = oracle.backward(X, layers, 2 * g1 - 3 * g2, EPS)
    np.testing.assert_allclose(d3, 2 * d1 - 3 * d2, rtol=1e-11, atol=1e-12)
    for n in range(2):
        for name in p3[n]:
            np.testing.assert_allclose(p3[n][name], 2 * p1[n][name] - 3 * p2[n][name], rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------- mixing

@pytest.mark.parametrize("T,D", [(4, 8), (3, 12), (8, 8), (5, 20)])
def test_mix_backward_is_the_adjoint_and_equals_the_mix(T, D):
    """<P x, g> = <x, P^T g>; P is a symmetric permutation, so P^T g = P g."""
    rng = np.random.default_rng(T * D)
    x = rng.standard_normal((2, T, D))
    g = rng.standard_normal((2, T, D))
    lhs = float((oracle.token_mix(x) * g).sum())
    rhs = float((x * oracle.token_mix_backward(g)).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    np.testing.assert_array_equal(oracle.token_mix_backward(g), oracle.token_mix(g))


def test_mix_backward_returns_each_coordinate_to_its_source():
    """Label coordinates by their own index: P^T sends the mixed labels back home."""
    T, D = 4, 8
    labels = np.arange(T * D, dtype=np.float64).reshape(T, D)
    np.testing.assert_array_equal(oracle.token_mix_backward(oracle.token_mix(labels)), labels)


# --------------------------------------------------------------------- GELU'

def test_gelu_grad_matches_difference_quotients_of_gelu():
    u = np.linspace(-6, 6, 97)
    h = 1e-5
    num = (oracle.gelu(u + h) - oracle.gelu(u - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_grad(u), num, rtol=0, atol=1e-9)


def test_gelu_grad_closed_forms():
    assert oracle.gelu_grad(0.0) == 0.5                       # Phi(0) = 1/2
    np.testing.assert_allclose(oracle.gelu_grad(np.array([12.0, -12.0])), [1.0, 0.0], atol=1e-15)
    # GELU'(u) + GELU'(-u) = 1: Phi(u) + Phi(-u) = 1 and the u phi(u) terms cancel
    u = np.linspace(-5, 5, 41)
    np.testing.assert_allclose(oracle.gelu_grad(u) + oracle.gelu_grad(-u), 1.0, atol=1e-15)
    # matches torch's exact-GELU autograd
    ut = torch.tensor(u, requires_grad=True)
    F.gelu(ut, approximate="none").sum().backward()
    np.testing.assert_allclose(oracle.gelu_grad(u), ut.grad.numpy(), rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------- LayerNorm

def test_layer_norm_backward_row_sums_vanish_and_match_autograd():
    """LN(r + c) = LN(r), so every row of dR sums to zero; values match torch autograd."""
    rng = np.random.default_rng(15)
    R = 2 * rng.standard_normal((7, 10)) + 1
    gam, bet = 1 + 0.3 * rng.standard_normal(10), 0.3 * rng.standard_normal(10)
    G = rng.standard_normal((7, 10))
    dR, dg, db = oracle.layer_norm_backward(R, gam, G, EPS)
    np.testing.assert_allclose(dR.sum(axis=-1), 0.0, atol=1e-13)
    Rt = torch.tensor(R, requires_grad=True)
    gt = torch.tensor(gam, requires_grad=True)
    bt = torch.tensor(bet, requires_grad=True)
    (F.layer_norm(Rt, (10,), gt, bt, EPS) * torch.tensor(G)).sum().backward()
    np.testing.assert_allclose(dR, Rt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_layer_norm_backward_scale_invariance_without_eps():
    """With eps = 0, LN(a r) = LN(r) for a > 0, so dR is orthogonal to r - mean(r)."""
    rng = np.random.default_rng(16)
    R = rng.standard_normal((5, 9))
    G = rng.standard_normal((5, 9))
    dR, _, _ = oracle.layer_norm_backward(R, np.ones(9), G, 0.0)
    Rc = R - R.mean(axis=-1, keepdims=True)
    np.testing.assert_allclose((dR * Rc).sum(axis=-1), 0.0, atol=1e-12)


# ---------------------------------------------------------------------- PFFN

def _mlp_grads(x, W1, b1, W2, b2, gv):
    """Autograd of a textbook Linear-GELU-Linear (torch's Linear: weight is out x in)."""
    xt = torch.tensor(x, requires_grad=True)
    w1, c1 = torch.tensor(W1.T.copy(), requires_grad=True), torch.tensor(b1, requires_grad=True)
    w2, c2 = torch.tensor(W2.T.copy(), requires_grad=True), torch.tensor(b2, requires_grad=True)
    v = F.linear(F.gelu(F.linear(xt, w1, c1), approximate="none"), w2, c2)
    (v * torch.tensor(gv)).sum().backward()
    return xt.grad.numpy(), w1.grad.numpy().T, c1.grad.numpy(), w2.grad.numpy().T, c2.grad.numpy()


def test_pffn_backward_with_equal_weights_is_one_mlp_backward():
    rng = np.random.default_rng(17)
    B, T, D, k = 5, 3, 6, 2
    W1 = rng.standard_normal((D, k * D)) / np.sqrt(D)
    W2 = rng.standard_normal((k * D, D)) / np.sqrt(k * D)
    b1, b2 = 0.2 * rng.standard_normal(k * D), 0.2 * rng.standard_normal(D)
    S = rng.standard_normal((B, T, D))
    GV = rng.standard_normal((B, T, D))
    rep = lambda a: np.repeat(a[None], T, 0)  # noqa: E731
    GS, dW1, db1, dW2, db2 = oracle.pffn_backward(S, rep(W1), rep(b1), rep(W2), rep(b2), GV)
    gx, gW1, gb1, gW2, gb2 = _mlp_grads(S.reshape(-1, D), W1, b1, W2, b2, GV.reshape(-1, D))
    np.testing.assert_allclose(GS, gx.reshape(B, T, D), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dW1.sum(0), gW1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(db1.sum(0), gb1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dW2.sum(0), gW2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(db2.sum(0), gb2, rtol=1e-11, atol=1e-12)


def test_pffn_backward_is_a_block_diagonal_mlp_backward():
    """Per-token weights = one MLP on the flattened row with block-diagonal weights; the
    diagonal blocks of that MLP's weight gradients are the per-token gradients."""
    rng = np.random.default_rng(18)
    B, T, D, k = 4, 3, 4, 2
    W1 = rng.standard_normal((T, D, k * D)) / np.sqrt(D)
    W2 = rng.standard_normal((T, k * D, D)) / np.sqrt(k * D)
    b1, b2 = 0.2 * rng.standard_normal((T, k * D)), 0.2 * rng.standard_normal((T, D))
    S = rng.standard_normal((B, T, D))
    GV = rng.standard_normal((B, T, D))
    GS, dW1, db1, dW2, db2 = oracle.pffn_backward(S, W1, b1, W2, b2, GV)
    bd1 = torch.block_diag(*[torch.tensor(w) for w in W1]).numpy()
    bd2 = torch.block_diag(*[torch.tensor(w) for w in W2]).numpy()
    gx, gW1, gb1, gW2, gb2 = _mlp_grads(S.reshape(B, -1), bd1, b1.reshape(-1), bd2, b2.reshape(-1),
                                        GV.reshape(B, -1))
    np.testing.assert_allclose(GS, gx.reshape(B, T, D), rtol=1e-11, atol=1e-12)
    kD = k * D
    for t in range(T):
        np.testing.assert_allclose(dW1[t], gW1[t * D:(t + 1) * D, t * kD:(t + 1) * kD], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dW2[t], gW2[t * kD:(t + 1) * kD, t * D:(t + 1) * D], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(db1, gb1.reshape(T, kD), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(db2, gb2.reshape(T, D), rtol=1e-11, atol=1e-12)


def test_moe_block_has_no_backward():
    rng = np.random.default_rng(19)
    p = _params(rng, 2, 4, 2, 1)[0]
    p["Wg"] = np.zeros((2, 4, 2))
    with pytest.raises(NotImplementedError):
        oracle.block_backward(rng.standard_normal((1, 2, 4)), p, EPS, rng.standard_normal((1, 2, 4)))


# ----------------------------------------------------------- prediction head

def test_prediction_head_worked_example():
    """[exp1] 6.4: o, w, b printed to 4 decimals; z, p, loss and dloss/dz computed by the
    page from full-precision values.  Rounding o and w to 4 decimals moves z by at most
    sum|w| * 5e-5 + sum|o| * 5e-5 + 5e-5 < 3e-4."""
    g = read("prediction_head_example.txt")
    z, p, loss, dz, do = oracle.bce_logit_head(g["o"], g["w"][0], g["b"][0, 0], g["y"][0])
    assert abs(z[0] - g["z"][0, 0]) < 3e-4
    assert abs(p[0] - g["p"][0, 0]) < 1e-4
    assert abs(loss[0] - g["loss"][0, 0]) < 2e-4
    assert abs(dz[0] - g["dz"][0, 0]) < 1e-4
    np.testing.assert_allclose(do[0], dz[0] * g["w"][0], rtol=1e-15)
    # the page's own consistency: dz = p - y with y = 1, and loss = -log p
    assert abs(g["dz"][0, 0] - (g["p"][0, 0] - 1.0)) < 2e-6
    assert abs(g["loss"][0, 0] + np.log(g["p"][0, 0])) < 2e-6


def test_prediction_head_gradient_matches_autograd():
    rng = np.random.default_rng(20)
    o, w, y = rng.standard_normal((6, 5)), rng.standard_normal(5), rng.integers(0, 2, 6).astype(float)
    z, p, loss, dz, do = oracle.bce_logit_head(o, w, 0.3, y)
    ot = torch.tensor(o, requires_grad=True)
    zt = ot @ torch.tensor(w) + 0.3
    F.binary_cross_entropy_with_logits(zt, torch.tensor(y), reduction="sum").backward()
    np.testing.assert_allclose(do, ot.grad.numpy(), rtol=1e-12, atol=1e-14)
