"""fp64 CPU oracle of the RankMixer block backward.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this module.  It shares nothing with the GPU library, and the GPU library never
imports it.

The gradients are the ones the tutorial page writes out for one sample, "RankMixer 详解
（1）：特征分组与完整计算流程" (jackknifer.me), section 5.2:
  * mean pool: every row of X_L receives g_o / T;
  * per-token FFN: g_a = g_v W2^T, g_u = g_a * GELU'(u), g_s = g_u W1^T, with
    GELU'(u) = Phi(u) + u phi(u); weight gradients a^T g_v, s^T g_u, bias gradients
    g_v, g_u;
  * LayerNorm: with r_hat = (r - mu) / sqrt(var + eps) and q = g * gamma,
    dr = (q - mean(q) - r_hat * mean(q * r_hat)) / sqrt(var + eps);
    dgamma = g * r_hat, dbeta = g;
  * Token Mixing: the input receives P^T g; before the first LayerNorm the residual adds
    the direct path, so dX = (P^T + I) g.
Section 5.2 also states that batch gradients add up over samples (or average, as the
loss does): here they are summed over samples, and over the T rows that share one
LayerNorm's gamma and beta.  The caller scales g_o for a mean loss.

The forward intermediates are recomputed from the inputs, block by block, with the
forward oracle's own functions (``rmx_oracle``); nothing is cached between calls.
The Sparse-MoE variant has no backward here.

Pinned by tests/test_oracle_backward.py: central finite differences of the forward
oracle, the adjoint identity of the mixing permutation, a shared-weights FFN against a
library autograd of a textbook MLP, closed forms of GELU', LayerNorm invariances, and
the page's worked prediction-head numbers (section 6.4).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from . import rmx_oracle as fwd

__all__ = ["gelu_grad", "layer_norm_backward", "token_mix_backward", "pffn_backward",
           "block_backward", "backward", "bce_logit_head"]

_PARAMS = ("W1", "b1", "W2", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def gelu_grad(u) -> np.ndarray:
    """Derivative of the exact GELU: Phi(u) + u phi(u), phi the standard normal density
    ([exp1] 5.2)."""
    u = _f64(u)
    Phi = 0.5 * (1.0 + erf(u / np.sqrt(2.0)))
    phi = np.exp(-0.5 * u * u) / np.sqrt(2.0 * np.pi)
    return Phi + u * phi


def layer_norm_backward(R, gamma, G, eps: float):
    """Backward of the row LayerNorm over the last axis ([exp1] 5.2).

    R: the LayerNorm input rows; G: the gradient its output receives (same shape).
    Returns (dR, dgamma, dbeta) with dgamma, dbeta summed over every row."""
    R, G, gamma = _f64(R), _f64(G), _f64(gamma)
    mu = R.mean(axis=-1, keepdims=True)
    var = ((R - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    rhat = (R - mu) * rstd
    q = G * gamma
    dR = (q - q.mean(axis=-1, keepdims=True) - rhat * (q * rhat).mean(axis=-1, keepdims=True)) * rstd
    D = R.shape[-1]
    dgamma = (G * rhat).reshape(-1, D).sum(axis=0)
    dbeta = G.reshape(-1, D).sum(axis=0)
    return dR, dgamma, dbeta


def token_mix_backward(G) -> np.ndarray:
    """P^T g for the Token Mixing permutation P over the last two axes ([exp1] 5.2).

    The forward copies X[t, h*q + r] to out[h, t*q + r]; its transpose returns every
    gradient coordinate to the input coordinate it was copied from."""
    G = _f64(G)
    T, D = G.shape[-2], G.shape[-1]
    if D % T:
        raise ValueError(f"D={D} is not divisible by H=T={T}")
    q = D // T
    dX = np.zeros_like(G)
    for h in range(T):
        for t in range(T):
            dX[..., t, h * q:(h + 1) * q] += G[..., h, t * q:(t + 1) * q]
    return dX


def pffn_backward(S, W1, b1, W2, b2, GV):
    """Backward of the per-token FFN v_t = GELU(s_t W1[t] + b1[t]) W2[t] + b2[t]
    ([exp1] 5.2; forward [paper] 3.3.2 eq (6)-(7)).

    S[B, T, D] the FFN input, GV[B, T, D] the gradient of its output.  Returns
    (GS, dW1, db1, dW2, db2): the gradient of S through the FFN only (the residual path is
    the caller's) and the weight gradients summed over the batch."""
    S, GV = _f64(S), _f64(GV)
    B, T, D = S.shape
    GS = np.empty_like(S)
    dW1, db1, dW2, db2 = [], [], [], []
    for t in range(T):
        w1, w2 = _f64(W1[t]), _f64(W2[t])
        U = S[:, t, :] @ w1 + _f64(b1[t])
        A = fwd.gelu(U)
        gv = GV[:, t, :]
        ga = gv @ w2.T
        gu = ga * gelu_grad(U)
        GS[:, t, :] = gu @ w1.T
        dW2.append(A.T @ gv)
        db2.append(gv.sum(axis=0))
        dW1.append(S[:, t, :].T @ gu)
        db1.append(gu.sum(axis=0))
    return GS, np.stack(dW1), np.stack(db1), np.stack(dW2), np.stack(db2)


def block_backward(X, p: dict, eps: float, GX):
    """Backward of one dense block X' = LN2(PFFN(S) + S), S = LN1(TokenMixing(X) + X)
    ([paper] 3.1 eq (1); gradients [exp1] 5.2).

    X[B, T, D] the block input, GX the gradient of its output X'.  Returns (dX, grads)
    with grads a dict of the parameter gradients named like the parameters."""
    if "Wg" in p:
        raise NotImplementedError("the Sparse-MoE block has no backward")
    X, GX = _f64(X), _f64(GX)
    R1 = fwd.token_mix(X) + X
    S = fwd.layer_norm(R1, p["ln1_g"], p["ln1_b"], eps)
    V = fwd.pffn(S, p["W1"], p["b1"], p["W2"], p["b2"])
    R2 = V + S
    GR2, dg2, db2n = layer_norm_backward(R2, p["ln2_g"], GX, eps)
    GS_ffn, dW1, db1, dW2, db2 = pffn_backward(S, p["W1"], p["b1"], p["W2"], p["b2"], GR2)
    GS = GS_ffn + GR2                       # the second residual passes GR2 straight to S
    GR1, dg1, db1n = layer_norm_backward(R1, p["ln1_g"], GS, eps)
    dX = GR1 + token_mix_backward(GR1)      # (P^T + I) g
    grads = {"W1": dW1, "b1": db1, "W2": dW2, "b2": db2,
             "ln1_g": dg1, "ln1_b": db1n, "ln2_g": dg2, "ln2_b": db2n}
    return dX, grads


def backward(X, layers: list, g_o, eps: float = 1e-5):
    """Gradients of a loss through L stacked dense blocks and the mean pool.

    X[B, T, D] the stack's input, g_o[B, D] the gradient of the pooled output o.  Every
    row of X_L receives g_o / T ([exp1] 5.2); the blocks are then walked from the last to
    the first, each recomputing its own forward from its input.  Returns
    (dX[B, T, D], [grads of block 1, ..., grads of block L])."""
    X, g_o = _f64(X), _f64(g_o)
    B, T, D = X.shape
    inputs = []
    for p in layers:
        inputs.append(X)
        X, _ = fwd.block(X, p, eps)
    G = np.broadcast_to(g_o[:, None, :] / T, (B, T, D)).copy()
    grads = [None] * len(layers)
    for n in range(len(layers) - 1, -1, -1):
        G, grads[n] = block_backward(inputs[n], layers[n], eps, G)
    return G, grads


def bce_logit_head(o, w, b, y):
    """The linear prediction head and binary cross-entropy of [exp1] 5.1-5.2:
    z = o w + b, p = sigmoid(z), loss = -y log p - (1 - y) log(1 - p), and the
    gradients dloss/dz = p - y and dloss/do = (p - y) w.
    o[B, D], w[D], b scalar, y[B] in {0, 1}.  Returns (z, p, loss, dz, do)."""
    o, w, y = _f64(o), _f64(w), _f64(y)
    z = o @ w + float(b)
    p = 1.0 / (1.0 + np.exp(-z))
    loss = -y * np.log(p) - (1.0 - y) * np.log(1.0 - p)
    dz = p - y
    return z, p, loss, dz, dz[:, None] * w[None, :]
