"""Seeded synthetic inputs for the RankMixer block forward.

This module is shared by the fp64 oracle tests and by the GPU tests / benchmark. It
holds none of the method's arithmetic: only random draws, scaling of the draws by a
standard deviation, zeroing of whole token rows, and rounding of the values to the
storage dtype (bf16, round-to-nearest-even). Every array it returns is float32 on the
host; for bf16 workloads each value is already exactly representable in bf16, so that
``torch.from_numpy(a).to(torch.bfloat16)`` is exact and the oracle's fp64 upcast sees
the very same numbers as the GPU.

Recipe (one substream per tensor slice, so slices can be drawn lazily and in
parallel): the slice (kind, layer, token, expert) of a tensor is drawn from
``numpy.random.Generator(PCG64(SeedSequence([seed, kind, layer, token, expert])))`` as
float32 standard normals, multiplied by the float32 standard deviation, and rounded to
the dtype. X is drawn in blocks of 64 samples (substream ``[seed, KIND_X, block]``).
Shapes follow the pages' parameter shapes (RankMixer paper translation, section 3.3.2,
eq (7)): W1[t] is D x kD, W2[t] is kD x D, the row-vector convention ``x W + b``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Substream kind codes (part of the recipe: changing one changes every input).
KIND_X, KIND_MASK = 1, 2
KIND_W1, KIND_B1, KIND_W2, KIND_B2 = 10, 11, 12, 13
KIND_G1, KIND_BE1, KIND_G2, KIND_BE2 = 20, 21, 22, 23
KIND_WG, KIND_WE1, KIND_BEXP1, KIND_WE2, KIND_BEXP2 = 30, 31, 32, 33, 34
KIND_E, KIND_WP, KIND_BP = 40, 41, 42
KIND_GOUT = 50
KIND_WQ, KIND_WK, KIND_WV = 60, 61, 62

X_BLOCK = 64


@dataclass(frozen=True)
class Config:
    """One workload: shapes, dtype and the distributions of its inputs."""
    name: str
    B: int
    T: int
    D: int
    k: int
    L: int
    dtype: str = "bf16"          # "fp32" or "bf16": dtype of X, weights and activations
    ln_init: str = "jitter"      # "unit": gamma=1, beta=0; "jitter": gamma~1+0.02N, beta~0.02N
    bias_std: float = 0.0        # 0 -> all biases are zero
    zero_frac: float = 0.0       # fraction of (b, t) token rows of X set to zero
    E: int = 0                   # Sparse-MoE experts per token (0 = dense per-token FFN)
    moe_hidden: int = 0          # hidden width of one expert
    eps: float = 1e-5
    routing: str = "mix"         # "mix": Token Mixing; "attention": the self-attention comparator

    @property
    def H(self) -> int:
        return self.T

    @property
    def kD(self) -> int:
        return self.k * self.D

    def with_(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


# The five workloads.  Sizes and distributions as the build's specification states them.
TINY = Config("tiny", B=8, T=4, D=8, k=2, L=1, dtype="fp32", ln_init="unit")
M100 = Config("rankmixer-100m", B=512, T=16, D=768, k=4, L=2, dtype="bf16")
B1 = Config("rankmixer-1b", B=2048, T=32, D=1536, k=4, L=2, dtype="bf16")
SWEEP_BATCHES = (64, 256, 1024, 4096, 16384)
SWEEP = B1.with_(name="rankmixer-1b-sweep", zero_frac=0.10)
MOE = Config("rankmixer-1b-moe", B=2048, T=32, D=1536, k=4, L=2, dtype="bf16",
             E=8, moe_hidden=3072)
# The routing comparator of the pages' ablation: the same blocks with self-attention in place
# of Token Mixing (the pages ran it at the 100M scale).
M100_ATTN = M100.with_(name="rankmixer-100m-attention", routing="attention")
B1_ATTN = B1.with_(name="rankmixer-1b-attention", routing="attention")
CONFIGS = {c.name: c for c in (TINY, M100, B1, SWEEP, MOE, M100_ATTN, B1_ATTN)}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    out = ((bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)).view(np.float32)
    return out


def _gen(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def _normal(seed: int, key, shape, std: float, mean: float = 0.0) -> np.ndarray:
    a = _gen(seed, *key).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclass
class Inputs:
    """Host copies of one workload's inputs.  Per-layer tensors are stacked over L."""
    cfg: Config
    X: np.ndarray                       # [B, T, D]
    W1: np.ndarray                      # [L, T, D, kD]
    b1: np.ndarray                      # [L, T, kD]
    W2: np.ndarray                      # [L, T, kD, D]
    b2: np.ndarray                      # [L, T, D]
    ln1_g: np.ndarray                   # [L, D]
    ln1_b: np.ndarray
    ln2_g: np.ndarray
    ln2_b: np.ndarray
    moe: dict = field(default_factory=dict)   # Wg [L,T,D,E], We1 [L,T,E,D,h], be1, We2, be2
    attn: dict = field(default_factory=dict)  # Wq, Wk, Wv [L, D, D] (self-attention routing)

    def layer(self, n: int) -> dict:
        """Parameters of block n (0-based) as a dict of views."""
        d = dict(W1=self.W1[n], b1=self.b1[n], W2=self.W2[n], b2=self.b2[n],
                 ln1_g=self.ln1_g[n], ln1_b=self.ln1_b[n],
                 ln2_g=self.ln2_g[n], ln2_b=self.ln2_b[n])
        for key, arr in self.moe.items():
            d[key] = arr[n]
        for key, arr in self.attn.items():
            d[key] = arr[n]
        return d

    def layers(self) -> list:
        return [self.layer(n) for n in range(self.cfg.L)]


def _fill_slices(out: np.ndarray, draw, keys, dtype: str) -> None:
    """out[i] = draw(keys[i]) for every i, drawn in parallel threads."""
    def one(i):
        v = draw(keys[i])
        out[i] = round_bf16(v) if dtype == "bf16" else v
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(len(keys))))


def make_x(cfg: Config, seed: int = 0, B: int | None = None) -> np.ndarray:
    """Token batch X[B, T, D] ~ N(0, 1), with cfg.zero_frac of its token rows zeroed."""
    B = cfg.B if B is None else B
    T, D = cfg.T, cfg.D
    X = np.empty((B, T, D), dtype=np.float32)
    nblk = (B + X_BLOCK - 1) // X_BLOCK

    def one(i):
        lo, hi = i * X_BLOCK, min(B, (i + 1) * X_BLOCK)
        v = _normal(seed, (KIND_X, i), (hi - lo, T, D), 1.0)
        X[lo:hi] = round_bf16(v) if cfg.dtype == "bf16" else v
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(nblk)))
    if cfg.zero_frac > 0.0:
        nzero = int(round(cfg.zero_frac * B * T))
        rows = _gen(seed, KIND_MASK).permutation(B * T)[:nzero]
        X.reshape(B * T, D)[rows] = 0.0
    return X


def make_inputs(cfg: Config, seed: int = 0, B: int | None = None) -> Inputs:
    """All inputs of one workload: X and the weights of its L blocks (float32 arrays)."""
    L, T, D, kD = cfg.L, cfg.T, cfg.D, cfg.kD
    dt = cfg.dtype
    X = make_x(cfg, seed, B)

    def stacked(kind, shape_per_token, std, per_token=True, mean=0.0):
        if per_token:
            out = np.empty((L, T) + shape_per_token, dtype=np.float32)
            keys = [(kind, l, t) for l in range(L) for t in range(T)]
            flat = out.reshape((L * T,) + shape_per_token)
            _fill_slices(flat, lambda key: _normal(seed, key, shape_per_token, std, mean), keys, dt)
        else:
            out = np.empty((L,) + shape_per_token, dtype=np.float32)
            keys = [(kind, l) for l in range(L)]
            _fill_slices(out, lambda key: _normal(seed, key, shape_per_token, std, mean), keys, dt)
        return out

    def zeros_or(kind, shape, per_token=True):
        if cfg.bias_std == 0.0:
            return np.zeros(((L, T) if per_token else (L,)) + shape, dtype=np.float32)
        return stacked(kind, shape, cfg.bias_std, per_token)

    W1 = stacked(KIND_W1, (D, kD), 1.0 / np.sqrt(D))
    b1 = zeros_or(KIND_B1, (kD,))
    W2 = stacked(KIND_W2, (kD, D), 1.0 / np.sqrt(kD))
    b2 = zeros_or(KIND_B2, (D,))
    if cfg.ln_init == "unit":
        ones = np.ones((L, D), dtype=np.float32)
        zero = np.zeros((L, D), dtype=np.float32)
        g1, be1, g2, be2 = ones, zero, ones.copy(), zero.copy()
    else:
        g1 = stacked(KIND_G1, (D,), 0.02, per_token=False, mean=1.0)
        be1 = stacked(KIND_BE1, (D,), 0.02, per_token=False)
        g2 = stacked(KIND_G2, (D,), 0.02, per_token=False, mean=1.0)
        be2 = stacked(KIND_BE2, (D,), 0.02, per_token=False)
    inp = Inputs(cfg, X, W1, b1, W2, b2, g1, be1, g2, be2)
    if cfg.E > 0:
        E, h = cfg.E, cfg.moe_hidden
        inp.moe = dict(
            Wg=stacked(KIND_WG, (D, E), 1.0 / np.sqrt(D)),
            We1=_stacked_expert(cfg, seed, KIND_WE1, (D, h), 1.0 / np.sqrt(D)),
            be1=_expert_bias(cfg, seed, KIND_BEXP1, (h,)),
            We2=_stacked_expert(cfg, seed, KIND_WE2, (h, D), 1.0 / np.sqrt(h)),
            be2=_expert_bias(cfg, seed, KIND_BEXP2, (D,)),
        )
    if cfg.routing == "attention":
        inp.attn = {name: stacked(kind, (D, D), 1.0 / np.sqrt(D), per_token=False)
                    for name, kind in (("Wq", KIND_WQ), ("Wk", KIND_WK), ("Wv", KIND_WV))}
    return inp


def _stacked_expert(cfg, seed, kind, shape, std):
    L, T, E = cfg.L, cfg.T, cfg.E
    out = np.empty((L, T, E) + shape, dtype=np.float32)
    keys = [(kind, l, t, e) for l in range(L) for t in range(T) for e in range(E)]
    _fill_slices(out.reshape((L * T * E,) + shape),
                 lambda key: _normal(seed, key, shape, std), keys, cfg.dtype)
    return out


def _expert_bias(cfg, seed, kind, shape):
    L, T, E = cfg.L, cfg.T, cfg.E
    if cfg.bias_std == 0.0:
        return np.zeros((L, T, E) + shape, dtype=np.float32)
    return _stacked_expert(cfg, seed, kind, shape, cfg.bias_std)



# Tokenisation projection workload: the concatenated embedding of the 1B shape's input.
# The pages give no per-token slice width d for it; 512 is taken (a 16,384-wide
# concatenated embedding), d = D is covered by the tests.
TOKENIZE_D = 512


@dataclass
class TokenizeInputs:
    """Host copies of one tokenisation workload: E [B, T*d], Wp [T, d, D], bp [T, D]."""
    E: np.ndarray
    Wp: np.ndarray
    bp: np.ndarray


def make_tokenize_inputs(B: int, T: int, d: int, D: int, dtype: str = "bf16", seed: int = 0,
                         bias_std: float = 0.0) -> TokenizeInputs:
    """E ~ N(0, 1) drawn in blocks of 64 samples; Wp[t] ~ N(0, 1/d) (std = 1/sqrt(fan_in));
    bp[t] ~ N(0, bias_std^2) or zero.  Same per-slice substreams as make_inputs."""
    E = np.empty((B, T * d), dtype=np.float32)
    nblk = (B + X_BLOCK - 1) // X_BLOCK

    def one(i):
        lo, hi = i * X_BLOCK, min(B, (i + 1) * X_BLOCK)
        v = _normal(seed, (KIND_E, i), (hi - lo, T * d), 1.0)
        E[lo:hi] = round_bf16(v) if dtype == "bf16" else v
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(nblk)))
    Wp = np.empty((T, d, D), dtype=np.float32)
    _fill_slices(Wp, lambda key: _normal(seed, key, (d, D), 1.0 / np.sqrt(d)), [(KIND_WP, t) for t in range(T)],
                 dtype)
    bp = np.zeros((T, D), dtype=np.float32)
    if bias_std > 0.0:
        _fill_slices(bp, lambda key: _normal(seed, key, (D,), bias_std), [(KIND_BP, t) for t in range(T)], dtype)
    return TokenizeInputs(E=E, Wp=Wp, bp=bp)


def make_grad_out(B: int, D: int, seed: int = 0, rows=None) -> np.ndarray:
    """Upstream gradient of the pooled output for the backward pass, fp32 [B, D]: N(0, 1)
    in blocks of 64 samples (per-block substreams, like X).  rows: if given, only those
    samples keep their gradient, the others are zero."""
    G = np.empty((B, D), dtype=np.float32)
    nblk = (B + X_BLOCK - 1) // X_BLOCK
    for i in range(nblk):
        lo, hi = i * X_BLOCK, min(B, (i + 1) * X_BLOCK)
        G[lo:hi] = _normal(seed, (KIND_GOUT, i), (hi - lo, D), 1.0)
    if rows is not None:
        keep = np.zeros(B, dtype=bool)
        keep[np.asarray(rows)] = True
        G[~keep] = 0.0
    return G

