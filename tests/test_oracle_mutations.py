"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in the oracle (monkeypatching one function, on the CPU)
and checks that at least one pin of tests/test_oracle_pins.py then fails.
"""
import numpy as np
import pytest
from scipy.special import erf

import oracle
import oracle.rmx_oracle as ro
from tests import test_oracle_pins as pins

ORIG = {name: getattr(ro, name) for name in ("token_mix", "layer_norm", "gelu", "pffn", "moe_gates", "tokenize")}


def _mix_identity(X):
    return X.copy()


def _mix_reversed_heads(X):
    T, D = X.shape[-2:]
    q = D // T
    out = np.empty_like(X)
    for h in range(T):
        for t in range(T):
            out[..., h, t * q:(t + 1) * q] = X[..., t, h * q:(h + 1) * q][..., ::-1]
    return out


def _mix_tokens_reversed(X):
    T, D = X.shape[-2:]
    q = D // T
    out = np.empty_like(X)
    for h in range(T):
        for t in range(T):
            out[..., h, t * q:(t + 1) * q] = X[..., T - 1 - t, h * q:(h + 1) * q]
    return out


def _ln_unbiased(R, g, b, eps):
    R = np.asarray(R, dtype=np.float64)
    mu = R.mean(-1, keepdims=True)
    var = ((R - mu) ** 2).sum(-1, keepdims=True) / (R.shape[-1] - 1)
    return np.asarray(g) * (R - mu) / np.sqrt(var + eps) + np.asarray(b)


def _ln_eps_outside(R, g, b, eps):
    R = np.asarray(R, dtype=np.float64)
    mu = R.mean(-1, keepdims=True)
    var = ((R - mu) ** 2).mean(-1, keepdims=True)
    return np.asarray(g) * (R - mu) / (np.sqrt(var) + eps) + np.asarray(b)


def _ln_swapped_affine(R, g, b, eps):
    return ORIG["layer_norm"](R, b, g, eps)


def _gelu_tanh(u):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1 + np.tanh(np.sqrt(2 / np.pi) * (u + 0.044715 * u ** 3)))


def _gelu_wrong_scale(u):
    u = np.asarray(u, dtype=np.float64)
    return u * 0.5 * (1.0 + erf(u))


def _pffn_first_token_weights(S, W1, b1, W2, b2):
    T = np.asarray(S).shape[1]
    return ORIG["pffn"](S, [W1[0]] * T, [b1[0]] * T, [W2[0]] * T, [b2[0]] * T)


def _pffn_no_b2(S, W1, b1, W2, b2):
    return ORIG["pffn"](S, W1, b1, W2, [np.zeros_like(np.asarray(x)) for x in b2])


def _pffn_no_gelu(S, W1, b1, W2, b2):
    S = np.asarray(S, dtype=np.float64)
    V = np.empty_like(S)
    for t in range(S.shape[1]):
        V[:, t] = (S[:, t] @ W1[t] + b1[t]) @ W2[t] + b2[t]
    return V


def _gates_no_relu(S, Wg):
    S = np.asarray(S, dtype=np.float64)
    return np.stack([S[:, t] @ np.asarray(Wg[t]) for t in range(S.shape[1])], axis=1)


def _tok_transposed_slices(E, Wp, bp):
    # takes token t's coordinates strided by T instead of contiguous
    E = np.asarray(E, dtype=np.float64)
    T, d, D = np.shape(Wp)
    B = E.shape[0]
    Et = E.reshape(B, d, T).transpose(0, 2, 1).reshape(B, T * d)
    return ORIG["tokenize"](Et, Wp, bp)


def _tok_first_layer_shared(E, Wp, bp):
    T = np.shape(Wp)[0]
    return ORIG["tokenize"](E, [Wp[0]] * T, [bp[0]] * T)


def _tok_slice_shifted(E, Wp, bp):
    # off by one: token t starts at coordinate t*d + 1 (wrapping the last coordinate)
    E = np.roll(np.asarray(E, dtype=np.float64), -1, axis=1)
    return ORIG["tokenize"](E, Wp, bp)


MUTATIONS = {
    "tokenize_strided_slices": ("tokenize", _tok_transposed_slices),
    "tokenize_shared_first_layer": ("tokenize", _tok_first_layer_shared),
    "tokenize_slice_off_by_one": ("tokenize", _tok_slice_shifted),
    "mix_identity": ("token_mix", _mix_identity),
    "mix_reversed_within_head": ("token_mix", _mix_reversed_heads),
    "mix_tokens_reversed": ("token_mix", _mix_tokens_reversed),
    "ln_unbiased_variance": ("layer_norm", _ln_unbiased),
    "ln_eps_outside_sqrt": ("layer_norm", _ln_eps_outside),
    "ln_gamma_beta_swapped": ("layer_norm", _ln_swapped_affine),
    "gelu_tanh_approximation": ("gelu", _gelu_tanh),
    "gelu_missing_sqrt2": ("gelu", _gelu_wrong_scale),
    "pffn_shared_first_token": ("pffn", _pffn_first_token_weights),
    "pffn_dropped_b2": ("pffn", _pffn_no_b2),
    "pffn_dropped_gelu": ("pffn", _pffn_no_gelu),
    "moe_gate_without_relu": ("moe_gates", _gates_no_relu),
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
            for case in params[0].args[1]:
                calls.append((name, lambda fn=fn, case=case, argnames=argnames:
                              fn(**dict(zip(argnames, case)))))
        else:
            calls.append((name, fn))
    return calls


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    target, fake = MUTATIONS[mutation]
    monkeypatch.setattr(ro, target, fake)
    monkeypatch.setattr(oracle, target, fake)
    failed = []
    for name, call in _pin_calls():
        try:
            call()
        except (Exception, pytest.fail.Exception):
            failed.append(name)
    assert failed, f"no pin catches the planted mistake {mutation}"
