"""fp64 CPU oracle of the RankMixer block forward.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this module.  It shares nothing with the GPU library (no kernels, headers,
helpers or tables) and the GPU library never imports it.

Every step is the plain definition written out in fp64 NumPy, in the order the pages
give it; a library matmul and ``scipy.special.erf`` are the only library steps.

Pages cited (by title):
  [paper]  "RankMixer: Scaling Up Ranking Models in Industrial Recommenders"
           (Chinese translation, juejin.cn), sections 3.1-3.5, eq (1)-(12).
  [exp1]   "RankMixer 详解（1）：特征分组与完整计算流程" (jackknifer.me),
           sections 3.1, 3.3, 4.1, 5.1, 6.
  [uni]    "UniMixer: A Unified Architecture for Scaling Laws in Recommendation
           Systems" (Chinese translation, juejin.cn), eq (9), eq (10), Appendix A.

Readings taken where the pages leave a step open (each is listed in the design doc):
  * H = T, and D must be divisible by T ([paper] 3.3.1; [exp1] 3.1).
  * LayerNorm: biased variance (divide by D), eps inside the square root, one
    gamma/beta pair of length D per LayerNorm shared by all T rows ([exp1] 3.3).
  * GELU is the exact u * Phi(u) ([exp1] 4.1), not the tanh approximation.
  * Every block has its own parameters; the output is the mean over the T rows of
    X_L ([paper] 3.1 eq (1); [exp1] 5.1).
  * Sparse-MoE: gate g = ReLU(s W_g) with no bias and no renormalisation, an expert
    is a Linear-GELU-Linear of the eq (6)-(7) form, V = sum_e g_e * expert_e(s)
    summed in expert order ([paper] 3.4 eq (10)).
  * Self-attention routing (the comparator of [paper] 4.4, written out in [exp1] 3.4): one
    head, Q/K/V projections D x D shared by the T tokens, no output projection, scores
    scaled by 1 / sqrt(D); its output takes the place of TokenMixing(X) in the block.
  * Tokenisation: token i projects its own slice of the concatenated embedding with
    its own linear layer ([uni] eq (9) makes the layer token-specific; [paper] 3.2
    eq (2) and [exp1] 2 leave the sharing open), in the row-vector convention of the
    FFN: x_t = e[t*d:(t+1)*d] Wp[t] + bp[t], Wp[t] of shape d x D.

Pinned by tests/test_oracle_pins.py against the pages' worked examples, closed forms,
invariants, library special cases and brute force (tests/golden/ holds the pages'
printed values, each with its citation).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

__all__ = ["tokenize", "token_mix", "layer_norm", "gelu", "pffn", "moe_gates", "moe_pffn",
           "self_attention", "block", "forward"]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def tokenize(E: np.ndarray, Wp, bp) -> np.ndarray:
    """Tokenisation projection ([paper] 3.2 eq (2); [exp1] 2; [uni] eq (9)).

    E[B, T*d] is the concatenated feature embedding; token t takes the half-open slice
    E[:, t*d:(t+1)*d] (the first d coordinates go to the first token) and projects it to
    D dimensions with its own layer: X[:, t, :] = E[:, t*d:(t+1)*d] Wp[t] + bp[t],
    Wp[t] of shape d x D.  Returns X[B, T, D].
    """
    E = _f64(E)
    T, d, D = np.shape(Wp)
    B = E.shape[0]
    if E.shape[1] != T * d:
        raise ValueError(f"E has {E.shape[1]} columns, expected T*d = {T * d}")
    X = np.empty((B, T, D), dtype=np.float64)
    for t in range(T):
        X[:, t, :] = E[:, t * d:(t + 1) * d] @ _f64(Wp[t]) + _f64(bp[t])
    return X


def token_mix(X: np.ndarray) -> np.ndarray:
    """Multi-head Token Mixing with H = T over the last two axes of X[..., T, D].

    Split every token into H = T contiguous heads of q = D/T coordinates ([paper]
    eq (3)); mixed token h is the concatenation, in token order, of head h of every
    token ([paper] eq (4)).  In index form ([exp1] 3.1, 0-based here):
        out[h, t*q + r] = X[t, h*q + r].
    Pure data movement: values are copied, never rounded.
    """
    T, D = X.shape[-2], X.shape[-1]
    if D % T:
        raise ValueError(f"D={D} is not divisible by H=T={T}")
    q = D // T
    out = np.empty_like(X)
    for h in range(T):
        for t in range(T):
            out[..., h, t * q:(t + 1) * q] = X[..., t, h * q:(h + 1) * q]
    return out


def layer_norm(R: np.ndarray, gamma, beta, eps: float) -> np.ndarray:
    """LayerNorm of every row over its last axis ([exp1] 3.3):
    mu = mean(r), var = mean((r - mu)^2), out = gamma * (r - mu) / sqrt(var + eps) + beta."""
    R = _f64(R)
    mu = R.mean(axis=-1, keepdims=True)
    var = ((R - mu) ** 2).mean(axis=-1, keepdims=True)
    return _f64(gamma) * (R - mu) / np.sqrt(var + eps) + _f64(beta)


def gelu(u: np.ndarray) -> np.ndarray:
    """Exact GELU, u * Phi(u) with Phi the standard normal CDF ([exp1] 4.1)."""
    u = _f64(u)
    return u * 0.5 * (1.0 + erf(u / np.sqrt(2.0)))


def pffn(S: np.ndarray, W1, b1, W2, b2) -> np.ndarray:
    """Per-token FFN over S[B, T, D] ([paper] 3.3.2 eq (6)-(9)).

    Token t has its own weights: v_t = GELU(s_t W1[t] + b1[t]) W2[t] + b2[t], with
    W1[t] of shape D x kD and W2[t] of shape kD x D (row-vector convention, eq (7)).
    The weight slices are upcast to fp64 one token at a time.
    """
    S = _f64(S)
    B, T, D = S.shape
    V = np.empty_like(S)
    for t in range(T):
        U = S[:, t, :] @ _f64(W1[t]) + _f64(b1[t])
        A = gelu(U)
        V[:, t, :] = A @ _f64(W2[t]) + _f64(b2[t])
    return V


def moe_gates(S: np.ndarray, Wg) -> np.ndarray:
    """ReLU router of the Sparse-MoE PFFN ([paper] 3.4 eq (10)): G[b, t, e] = max(0, s_bt Wg[t])_e."""
    S = _f64(S)
    B, T, D = S.shape
    E = np.asarray(Wg[0]).shape[-1]
    G = np.empty((B, T, E))
    for t in range(T):
        G[:, t, :] = np.maximum(0.0, S[:, t, :] @ _f64(Wg[t]))
    return G


def moe_pffn(S: np.ndarray, Wg, We1, be1, We2, be2):
    """Sparse-MoE PFFN ([paper] 3.4 eq (10)): v = sum_e G_e * expert_e(s), expert_e(s) =
    GELU(s We1[t,e] + be1[t,e]) We2[t,e] + be2[t,e].  An expert whose gate is 0 adds
    nothing; the sum runs in expert order.  Returns (V, G)."""
    S = _f64(S)
    B, T, D = S.shape
    G = moe_gates(S, Wg)
    E = G.shape[-1]
    V = np.zeros_like(S)
    for t in range(T):
        for e in range(E):
            rows = np.nonzero(G[:, t, e] > 0.0)[0]
            if rows.size == 0:
                continue
            s = S[rows, t, :]
            y = gelu(s @ _f64(We1[t][e]) + _f64(be1[t][e])) @ _f64(We2[t][e]) + _f64(be2[t][e])
            V[rows, t, :] += G[rows, t, e][:, None] * y
    return V, G


def self_attention(X: np.ndarray, Wq, Wk, Wv) -> np.ndarray:
    """Single-head self-attention over the T tokens of each sample ([exp1] 3.4):
    Q = X Wq, K = X Wk, V = X Wv, out = softmax(Q K^T / sqrt(d_a)) V with the softmax along
    each row (over the keys).  X[..., T, D]; Wq, Wk of shape D x d_a, Wv of shape D x D
    (the output replaces TokenMixing(X), so it keeps width D)."""
    X = _f64(X)
    Q, K, V = X @ _f64(Wq), X @ _f64(Wk), X @ _f64(Wv)
    scores = Q @ np.swapaxes(K, -1, -2) / np.sqrt(Q.shape[-1])
    scores = scores - scores.max(axis=-1, keepdims=True)
    P = np.exp(scores)
    P /= P.sum(axis=-1, keepdims=True)
    return P @ V


def block(X: np.ndarray, p: dict, eps: float):
    """One RankMixer block ([paper] 3.1 eq (1), 3.3.1 eq (5)):
        S = LN1(TokenMixing(X) + X),   X' = LN2(PFFN(S) + S).
    p holds W1, b1, W2, b2, ln1_g, ln1_b, ln2_g, ln2_b (and Wg, We1, be1, We2, be2 for
    the Sparse-MoE variant).  With Wq, Wk, Wv in p the block is the routing comparator of
    [paper] 4.4 (self-attention between the tokens instead of Token Mixing):
        S = LN1(SelfAttention(X) + X).
    Returns (X', G) with G the MoE gates or None."""
    X = _f64(X)
    routed = self_attention(X, p["Wq"], p["Wk"], p["Wv"]) if "Wq" in p else token_mix(X)
    S = layer_norm(routed + X, p["ln1_g"], p["ln1_b"], eps)
    if "Wg" in p:
        V, G = moe_pffn(S, p["Wg"], p["We1"], p["be1"], p["We2"], p["be2"])
    else:
        V, G = pffn(S, p["W1"], p["b1"], p["W2"], p["b2"]), None
    return layer_norm(V + S, p["ln2_g"], p["ln2_b"], eps), G


def forward(X: np.ndarray, layers: list, eps: float = 1e-5):
    """L stacked blocks then the mean pool over tokens ([paper] 3.1; [exp1] 5.1).

    X: [B, T, D] (any float dtype; upcast to fp64).  layers: one parameter dict per
    block.  Returns (o[B, D], X_L[B, T, D], gates) where gates is a list holding each
    block's MoE gates [B, T, E] (None for a dense block)."""
    X = _f64(X)
    if X.ndim != 3:
        raise ValueError("X must be [B, T, D]")
    gates = []
    for p in layers:
        X, G = block(X, p, eps)
        gates.append(G)
    return X.mean(axis=1), X, gates
