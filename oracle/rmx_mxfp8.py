"""fp64 CPU oracle of the MXFP8 inference variant of the block forward.  TEST
INFRASTRUCTURE ONLY (imported by the tests and the benchmark's CPU-baseline leg, never by
the GPU library, with which it shares nothing).

The pages serve the model at a reduced precision because the core of the block is a few
large products and halving the operand width doubles the hardware peak ("RankMixer" paper
translation, section 4.6, eq (13) and its quantization item: fp16 inference).  On a part
whose bf16 and fp16 peaks are equal, the same step is 8-bit operands: the variant here
quantizes the operands of the two per-token products to MXFP8 as the OCP Microscaling
Formats (MX) Specification v1.0 defines it (a published format, not the pages'): every
block of 32 consecutive values along the reduction axis shares one power-of-two scale
X = 2^(floor(log2(amax)) - 8), 8 being the largest exponent of the FP8 E4M3 element format,
and each value is stored as the E4M3 number nearest to v / X (round to nearest, ties to even; E4M3 has 3 mantissa bits, exponent bias 7,
subnormals below 2^-6 in steps of 2^-9, largest finite 448; values beyond saturate to
+-448).  Where the quantization sits (a reading; the pages say nothing about it):
  * S, the LN1 output, along D (the K of the first product) for each (sample, token) row;
  * W1[t] and W2[t] along their K dimension (D and kD), for each output column;
  * H = GELU(U), along kD (the K of the second product), for each row;
  * everything else as the forward oracle: the residual S, LayerNorm, GELU, biases, the
    pool are unquantized.
``forward_mxfp8`` is that computation written out in fp64 with quantize-dequantize steps.
``mx_qdq`` is pinned in tests/test_oracle_mxfp8.py against the library's FP8 E4M3 cast,
closed forms and invariants; the parity tests compare the GPU variant with
``forward_mxfp8`` tightly and with the unquantized ``forward`` at a tolerance derived from
the format's precision.
"""
from __future__ import annotations

import numpy as np

from . import rmx_oracle as fwd

__all__ = ["e4m3_round", "mx_scale_exponent", "mx_qdq", "quantize_weights", "forward_mxfp8"]

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest E4M3 binade
MX_BLOCK = 32


def e4m3_round(v) -> np.ndarray:
    """Nearest FP8 E4M3 value (ties to even), saturating at +-448; exact in fp64."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    # binade exponent of |v| (frexp: a = m 2^e with m in [0.5, 1)); below 2^-6 the grid is
    # the subnormal step 2^-9
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    E = np.maximum(e - 1, -6)
    quantum = np.ldexp(1.0, E - 3)
    q = np.round(v / quantum) * quantum          # np.round: ties to even
    return np.clip(q, -E4M3_MAX, E4M3_MAX)


def mx_scale_exponent(amax) -> np.ndarray:
    """Shared exponent of an MX block: floor(log2(amax)) - 8, clamped to the E8M0 range
    [-127, 127]; an all-zero block takes -127."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    x = np.where(amax > 0, (e - 1) - E4M3_EMAX, -127)
    return np.clip(x, -127, 127).astype(np.int64)


def mx_qdq(x, axis: int = -1) -> np.ndarray:
    """Quantize x to MXFP8 E4M3 along `axis` (blocks of 32 consecutive values; the axis
    length must be a multiple of 32) and return the represented values in fp64."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    if n % MX_BLOCK:
        raise ValueError(f"axis length {n} is not a multiple of {MX_BLOCK}")
    blocks = x.reshape(*x.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    e = mx_scale_exponent(np.abs(blocks).max(axis=-1, keepdims=True))
    q = e4m3_round(np.ldexp(blocks, -e)) * np.ldexp(1.0, e)
    return np.moveaxis(q.reshape(x.shape), -1, axis)


def quantize_weights(layers: list, workers: int = 1) -> list:
    """mx_qdq of W1[t] and W2[t] along K (axis 0) for every block and token: a list over
    blocks of lists over tokens of (w1, w2).  The matrices are independent; `workers` > 1
    evaluates them on that many threads (the same function on the same values: the result
    does not depend on it)."""
    jobs = [(n, t) for n, p in enumerate(layers) for t in range(len(p["W1"]))]

    def one(job):
        n, t = job
        return mx_qdq(layers[n]["W1"][t], axis=0), mx_qdq(layers[n]["W2"][t], axis=0)

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            done = list(ex.map(one, jobs))
    else:
        done = [one(j) for j in jobs]
    out = [[None] * len(p["W1"]) for p in layers]
    for (n, t), wq in zip(jobs, done):
        out[n][t] = wq
    return out


def forward_mxfp8(X, layers: list, eps: float = 1e-5, wq: list | None = None):
    """The block stack and pool of ``rmx_oracle.forward`` with the products' operands
    quantized to MXFP8 as the module docstring states.  Dense blocks only.
    wq: the weights already passed through ``quantize_weights(layers)`` (optional; they are
    quantized here otherwise).  Returns (o[B, D], X_L[B, T, D])."""
    X = np.asarray(X, dtype=np.float64)
    for n, p in enumerate(layers):
        if "Wg" in p:
            raise NotImplementedError("the MXFP8 variant covers the dense per-token FFN")
        S = fwd.layer_norm(fwd.token_mix(X) + X, p["ln1_g"], p["ln1_b"], eps)
        Sq = mx_qdq(S, axis=-1)
        B, T, D = S.shape
        V = np.empty_like(S)
        for t in range(T):
            if wq is not None:
                w1, w2 = wq[n][t]
            else:
                w1 = mx_qdq(p["W1"][t], axis=0)
                w2 = mx_qdq(p["W2"][t], axis=0)
            H = fwd.gelu(Sq[:, t, :] @ w1 + np.asarray(p["b1"][t], dtype=np.float64))
            V[:, t, :] = mx_qdq(H, axis=-1) @ w2 + np.asarray(p["b2"][t], dtype=np.float64)
        X = fwd.layer_norm(V + S, p["ln2_g"], p["ln2_b"], eps)
    return X.mean(axis=1), X
