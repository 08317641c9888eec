"""The backward oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in the backward oracle (monkeypatching one function, on the
CPU) and checks that at least one pin of tests/test_oracle_backward.py then fails.
"""
import numpy as np
import pytest
from scipy.special import erf

import oracle
import oracle.rmx_backward as rb
from tests import test_oracle_backward as pins

ORIG = {name: getattr(rb, name) for name in ("layer_norm_backward", "gelu_grad", "token_mix_backward",
                                             "pffn_backward", "block_backward", "backward")}


def _ln_rows(R, eps):
    R = np.asarray(R, dtype=np.float64)
    mu = R.mean(-1, keepdims=True)
    rstd = 1 / np.sqrt(((R - mu) ** 2).mean(-1, keepdims=True) + eps)
    return R, mu, rstd, (R - mu) * rstd


def _ln_bwd_no_projection(R, gamma, G, eps):
    R, mu, rstd, rhat = _ln_rows(R, eps)
    q = np.asarray(G) * gamma
    D = R.shape[-1]
    return (q - q.mean(-1, keepdims=True)) * rstd, (G * rhat).reshape(-1, D).sum(0), np.reshape(G, (-1, D)).sum(0)


def _ln_bwd_no_gamma(R, gamma, G, eps):
    return ORIG["layer_norm_backward"](R, np.ones_like(np.asarray(gamma, dtype=np.float64)), G, eps)[0], \
        *ORIG["layer_norm_backward"](R, gamma, G, eps)[1:]


def _ln_bwd_dgamma_unnormalised(R, gamma, G, eps):
    dR, _, db = ORIG["layer_norm_backward"](R, gamma, G, eps)
    R, mu, _, _ = _ln_rows(R, eps)
    return dR, (np.asarray(G) * (R - mu)).reshape(-1, R.shape[-1]).sum(0), db


def _gelu_grad_cdf_only(u):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * (1 + erf(u / np.sqrt(2)))


def _gelu_grad_tanh(u):
    u = np.asarray(u, dtype=np.float64)
    c = np.sqrt(2 / np.pi)
    th = np.tanh(c * (u + 0.044715 * u ** 3))
    return 0.5 * (1 + th) + 0.5 * u * (1 - th ** 2) * c * (1 + 3 * 0.044715 * u ** 2)


def _mix_bwd_identity(G):
    return np.array(G, dtype=np.float64)


def _mix_bwd_reversed_tokens(G):
    G = np.asarray(G, dtype=np.float64)
    T, D = G.shape[-2:]
    q = D // T
    dX = np.zeros_like(G)
    for h in range(T):
        for t in range(T):
            dX[..., T - 1 - t, h * q:(h + 1) * q] += G[..., h, t * q:(t + 1) * q]
    return dX


def _pffn_bwd_token0_weights(S, W1, b1, W2, b2, GV):
    T = np.shape(S)[1]
    GS, dW1, db1, dW2, db2 = ORIG["pffn_backward"](S, [W1[0]] * T, [b1[0]] * T, [W2[0]] * T, [b2[0]] * T, GV)
    return GS, dW1, db1, dW2, db2


def _pffn_bwd_preactivation_in_dW2(S, W1, b1, W2, b2, GV):
    GS, dW1, db1, dW2, db2 = ORIG["pffn_backward"](S, W1, b1, W2, b2, GV)
    S, GV = np.asarray(S, dtype=np.float64), np.asarray(GV, dtype=np.float64)
    dW2 = np.stack([(S[:, t] @ np.asarray(W1[t]) + np.asarray(b1[t])).T @ GV[:, t] for t in range(S.shape[1])])
    return GS, dW1, db1, dW2, db2


def _block_bwd_no_second_residual(X, p, eps, GX):
    X, GX = np.asarray(X, dtype=np.float64), np.asarray(GX, dtype=np.float64)
    R1 = oracle.token_mix(X) + X
    S = oracle.layer_norm(R1, p["ln1_g"], p["ln1_b"], eps)
    R2 = oracle.pffn(S, p["W1"], p["b1"], p["W2"], p["b2"]) + S
    GR2, dg2, db2n = rb.layer_norm_backward(R2, p["ln2_g"], GX, eps)
    GS, dW1, db1, dW2, db2 = rb.pffn_backward(S, p["W1"], p["b1"], p["W2"], p["b2"], GR2)
    GR1, dg1, db1n = rb.layer_norm_backward(R1, p["ln1_g"], GS, eps)
    dX = GR1 + rb.token_mix_backward(GR1)
    return dX, {"W1": dW1, "b1": db1, "W2": dW2, "b2": db2,
                "ln1_g": dg1, "ln1_b": db1n, "ln2_g": dg2, "ln2_b": db2n}


def _block_bwd_no_first_residual(X, p, eps, GX):
    dX, grads = ORIG["block_backward"](X, p, eps, GX)
    X = np.asarray(X, dtype=np.float64)
    R1 = oracle.token_mix(X) + X
    S = oracle.layer_norm(R1, p["ln1_g"], p["ln1_b"], eps)
    R2 = oracle.pffn(S, p["W1"], p["b1"], p["W2"], p["b2"]) + S
    GR2 = rb.layer_norm_backward(R2, p["ln2_g"], GX, eps)[0]
    GS = rb.pffn_backward(S, p["W1"], p["b1"], p["W2"], p["b2"], GR2)[0] + GR2
    GR1 = rb.layer_norm_backward(R1, p["ln1_g"], GS, eps)[0]
    return rb.token_mix_backward(GR1), grads


def _backward_pool_sum(X, layers, g_o, eps=1e-5):
    T = np.shape(X)[1]
    return ORIG["backward"](X, layers, np.asarray(g_o) * T, eps)


MUTATIONS = {
    "ln_bwd_dropped_projection_term": ("layer_norm_backward", _ln_bwd_no_projection),
    "ln_bwd_forgot_gamma": ("layer_norm_backward", _ln_bwd_no_gamma),
    "ln_bwd_dgamma_without_rstd": ("layer_norm_backward", _ln_bwd_dgamma_unnormalised),
    "gelu_grad_cdf_only": ("gelu_grad", _gelu_grad_cdf_only),
    "gelu_grad_of_tanh_form": ("gelu_grad", _gelu_grad_tanh),
    "mix_bwd_identity": ("token_mix_backward", _mix_bwd_identity),
    "mix_bwd_reversed_tokens": ("token_mix_backward", _mix_bwd_reversed_tokens),
    "pffn_bwd_token0_weights": ("pffn_backward", _pffn_bwd_token0_weights),
    "pffn_bwd_preactivation_in_dW2": ("pffn_backward", _pffn_bwd_preactivation_in_dW2),
    "block_bwd_no_second_residual": ("block_backward", _block_bwd_no_second_residual),
    "block_bwd_no_first_residual": ("block_backward", _block_bwd_no_first_residual),
    "backward_pool_sum_not_mean": ("backward", _backward_pool_sum),
}


def _pin_calls():
    """Every pin as a zero-argument callable (parametrised pins at their first case)."""
    calls = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames = [a.strip() for a in params[0].args[0].split(",")]
            case = params[0].args[1][0]
            case = case if isinstance(case, tuple) else (case,)
            calls.append((name, lambda fn=fn, case=case, argnames=argnames: fn(**dict(zip(argnames, case)))))
        else:
            calls.append((name, fn))
    return calls


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_backward_mistake_is_caught(mutation, monkeypatch):
    target, fake = MUTATIONS[mutation]
    monkeypatch.setattr(rb, target, fake)
    monkeypatch.setattr(oracle, target, fake)
    failed = []
    for name, call in _pin_calls():
        try:
            call()
        except (Exception, pytest.fail.Exception):
            failed.append(name)
    assert failed, f"no pin catches the planted mistake {mutation}"
