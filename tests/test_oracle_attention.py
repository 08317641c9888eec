"""Pins of the self-attention routing comparator in the oracle (CPU only).

[paper] 4.4 compares Token Mixing with self-attention between the tokens; [exp1] 3.4 writes
single-head attention out: Q = X Wq, K = X Wk, V = X Wv, softmax(Q K^T / sqrt(d_a)) V with
the softmax along each row.  Pinned by the library's scaled_dot_product_attention, closed
forms (zero query/key weights give the mean of V; a dominant diagonal gives V itself),
permutation equivariance, and the scalar twin of the whole block."""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle import brute

EPS = 1e-5


def _w(rng, D, s=1.0):
    return s * rng.standard_normal((D, D)) / np.sqrt(D)


def test_attention_matches_library_sdpa():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((5, 7, 12))
    Wq, Wk, Wv = _w(rng, 12, 2.0), _w(rng, 12, 2.0), _w(rng, 12)
    Xt = torch.tensor(X)
    ref = F.scaled_dot_product_attention(Xt @ torch.tensor(Wq), Xt @ torch.tensor(Wk), Xt @ torch.tensor(Wv))
    np.testing.assert_allclose(oracle.self_attention(X, Wq, Wk, Wv), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_zero_scores_average_the_values():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((3, 6, 8))
    Wv = _w(rng, 8)
    Z = np.zeros((8, 8))
    out = oracle.self_attention(X, Z, rng.standard_normal((8, 8)), Wv)
    np.testing.assert_allclose(out, np.broadcast_to((X @ Wv).mean(axis=1, keepdims=True), out.shape), rtol=1e-13, atol=1e-13)


def test_dominant_self_match_routes_each_token_to_itself():
    """Orthonormal token rows and Wq = Wk = c I: the score of a token with itself exceeds the
    others by c^2 / sqrt(D); for large c the attention is the identity and out = X Wv."""
    rng = np.random.default_rng(2)
    D, T = 8, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    X = Qm[:T][None]                                   # T orthonormal rows
    W = 12.0 * np.eye(D)
    Wv = _w(rng, D)
    np.testing.assert_allclose(oracle.self_attention(X, W, W, Wv), X @ Wv, atol=1e-12)


def test_attention_is_permutation_equivariant():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((2, 6, 10))
    Wq, Wk, Wv = _w(rng, 10), _w(rng, 10), _w(rng, 10)
    perm = rng.permutation(6)
    np.testing.assert_allclose(oracle.self_attention(X[:, perm], Wq, Wk, Wv),
                               oracle.self_attention(X, Wq, Wk, Wv)[:, perm], rtol=1e-12, atol=1e-12)


def test_attention_block_matches_scalar_twin():
    rng = np.random.default_rng(4)
    T, D, k, L = 4, 8, 2, 2
    X = rng.standard_normal((3, T, D))
    layers = []
    for _ in range(L):
        layers.append(dict(W1=rng.standard_normal((T, D, k * D)) / np.sqrt(D), b1=0.1 * rng.standard_normal((T, k * D)),
                           W2=rng.standard_normal((T, k * D, D)) / np.sqrt(k * D), b2=0.1 * rng.standard_normal((T, D)),
                           ln1_g=1 + 0.2 * rng.standard_normal(D), ln1_b=0.2 * rng.standard_normal(D),
                           ln2_g=1 + 0.2 * rng.standard_normal(D), ln2_b=0.2 * rng.standard_normal(D),
                           Wq=_w(rng, D, 2.0), Wk=_w(rng, D, 2.0), Wv=_w(rng, D)))
    o, XL, _ = oracle.forward(X, layers, EPS)
    for b in range(3):
        ob, xb, _ = brute.forward_sample(X[b], layers, EPS)
        np.testing.assert_allclose(XL[b], xb, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(o[b], ob, rtol=1e-11, atol=1e-11)
