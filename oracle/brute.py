"""Scalar-loop twin of the oracle for tiny shapes.  TEST INFRASTRUCTURE ONLY.

Written independently of rmx_oracle.py from the same definitions (pages cited by title
in rmx_oracle.py): every sum is an explicit Python loop over plain floats and GELU
uses ``math.erf``.  It exists to catch vectorisation mistakes in the NumPy oracle
(a wrong axis, a broadcast, a transposed operand); it is far too slow for anything
but a few hundred multiply-adds per sample.
"""
from __future__ import annotations

import math


def _mix(x, T, D):
    q = D // T
    out = [[0.0] * D for _ in range(T)]
    for h in range(T):
        for c in range(D):
            t, r = divmod(c, q)          # output column c of row h takes head h of token t
            out[h][c] = x[t][h * q + r]
    return out


def _ln_row(r, g, b, eps):
    n = len(r)
    mu = 0.0
    for v in r:
        mu += v
    mu /= n
    var = 0.0
    for v in r:
        var += (v - mu) * (v - mu)
    var /= n
    inv = 1.0 / math.sqrt(var + eps)
    return [g[j] * (r[j] - mu) * inv + b[j] for j in range(n)]


def _gelu(u):
    return u * 0.5 * (1.0 + math.erf(u / math.sqrt(2.0)))


def _linear(x, W, bias):
    # x: [n_in], W: [n_in][n_out] (row-vector convention), bias: [n_out]
    n_out = len(bias)
    y = []
    for j in range(n_out):
        acc = 0.0
        for i in range(len(x)):
            acc += x[i] * W[i][j]
        y.append(acc + bias[j])
    return y


def _attn(x, Wq, Wk, Wv):
    """Single-head self-attention of one sample x[T][D], scalar loops, softmax along keys."""
    T = len(x)
    zero = [0.0] * len(Wq[0])
    q = [_linear(x[t], Wq, zero) for t in range(T)]
    k = [_linear(x[t], Wk, zero) for t in range(T)]
    v = [_linear(x[t], Wv, [0.0] * len(Wv[0])) for t in range(T)]
    da = len(Wq[0])
    out = []
    for t in range(T):
        sc = [sum(q[t][i] * k[j][i] for i in range(da)) / math.sqrt(da) for j in range(T)]
        mx = max(sc)
        ex = [math.exp(c - mx) for c in sc]
        z = sum(ex)
        out.append([sum(ex[j] / z * v[j][c] for j in range(T)) for c in range(len(v[0]))])
    return out


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def forward_sample(x, layers, eps=1e-5):
    """One sample x[T][D] through all blocks; returns (o[D], x_L[T][D], gates)."""
    x = [[float(v) for v in row] for row in _tolist(x)]
    T, D = len(x), len(x[0])
    gates_all = []
    for p in layers:
        p = {key: _tolist(v) for key, v in p.items()}
        m = _attn(x, p["Wq"], p["Wk"], p["Wv"]) if "Wq" in p else _mix(x, T, D)
        s = [_ln_row([m[t][j] + x[t][j] for j in range(D)], p["ln1_g"], p["ln1_b"], eps)
             for t in range(T)]
        v = []
        gates = []
        for t in range(T):
            if "Wg" in p:
                E = len(p["Wg"][t][0])
                g = [max(0.0, sum(s[t][i] * p["Wg"][t][i][e] for i in range(D))) for e in range(E)]
                gates.append(g)
                acc = [0.0] * D
                for e in range(E):
                    if g[e] <= 0.0:
                        continue
                    hid = [_gelu(u) for u in _linear(s[t], p["We1"][t][e], p["be1"][t][e])]
                    y = _linear(hid, p["We2"][t][e], p["be2"][t][e])
                    for j in range(D):
                        acc[j] += g[e] * y[j]
                v.append(acc)
            else:
                hid = [_gelu(u) for u in _linear(s[t], p["W1"][t], p["b1"][t])]
                v.append(_linear(hid, p["W2"][t], p["b2"][t]))
        x = [_ln_row([v[t][j] + s[t][j] for j in range(D)], p["ln2_g"], p["ln2_b"], eps)
             for t in range(T)]
        gates_all.append(gates if gates else None)
    o = [sum(x[t][j] for t in range(T)) / T for j in range(D)]
    return o, x, gates_all


def tokenize_sample(e, Wp, bp):
    """One sample's concatenated embedding e[T*d] -> tokens x[T][D] with scalar loops:
    token t projects coordinates t*d .. t*d + d - 1 with its own Wp[t][d][D], bp[t][D]."""
    e = [float(v) for v in _tolist(e)]
    Wp, bp = _tolist(Wp), _tolist(bp)
    T = len(Wp)
    d = len(Wp[0])
    out = []
    for t in range(T):
        piece = e[t * d:(t + 1) * d]
        out.append(_linear(piece, Wp[t], bp[t]))
    return out
