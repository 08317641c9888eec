"""The attention pins catch plausible mistakes (CPU only): each case plants one mistake in
the oracle's self_attention and checks that a pin of tests/test_oracle_attention.py fails."""
import numpy as np
import pytest

import oracle
import oracle.rmx_oracle as ro
from tests import test_oracle_attention as pins


def _softmax(s, axis):
    s = s - s.max(axis=axis, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=axis, keepdims=True)


def _attn(X, Wq, Wk, Wv, scale=True, axis=-1, swap=False):
    X = np.asarray(X, dtype=np.float64)
    Q, K, V = X @ np.asarray(Wq), X @ np.asarray(Wk), X @ np.asarray(Wv)
    if swap:
        Q, K = K, Q
    s = Q @ np.swapaxes(K, -1, -2)
    if scale:
        s = s / np.sqrt(Q.shape[-1])
    return _softmax(s, axis) @ V


MUTATIONS = {
    "attn_unscaled_scores": lambda X, a, b, c: _attn(X, a, b, c, scale=False),
    "attn_softmax_over_queries": lambda X, a, b, c: _attn(X, a, b, c, axis=-2),
    "attn_keys_for_queries": lambda X, a, b, c: _attn(X, a, b, c, swap=True),
    "attn_values_unprojected": lambda X, a, b, c: _attn(X, a, b, np.eye(np.shape(c)[0])),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_attention_mistake_is_caught(mutation, monkeypatch):
    monkeypatch.setattr(ro, "self_attention", MUTATIONS[mutation])
    monkeypatch.setattr(oracle, "self_attention", MUTATIONS[mutation])
    failed = []
    for name in dir(pins):
        if name.startswith("test_"):
            try:
                getattr(pins, name)()
            except Exception:
                failed.append(name)
    assert failed, f"no pin catches {mutation}"
