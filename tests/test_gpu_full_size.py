"""Parity at the full sizes of the workloads, in the launch configuration the benchmark
times (weights prepared with rmx_pack_weights, a handle sized for the batch), against the
fp64 oracle on samples stratified over the products' 256-row tiles.

Samples are independent (mixing, LayerNorm and the per-token FFN never cross samples), so
the oracle's result for a sampled sample is exact in meaning at any batch size.  Every
sampled tile contributes its first and last row (the ragged edges) and seeded rows inside.
The Sparse-MoE routing lists are compared bit for bit with the gate values the same
forward wrote (RankMixer paper translation, section 3.4 eq (10): a variable number of
active experts per token), and their activity with the oracle's gates away from zero.
"""
import numpy as np
import pytest

import oracle
from rankmixer_block_forward_amd import synth
from tests.parity import check, check_moe_lists, run_gpu, run_oracle, sample_tiles, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_CACHE = {}


def _inputs(cfg, B=None):
    """Inputs of a workload, seed 0.  The weights of a seed depend only on the model's
    shapes (each slice has its own substream), so the dense 1B weights are drawn once and
    each batch size of the serving sweep draws only its X."""
    import dataclasses
    if cfg.E > 0:
        if "moe" not in _CACHE:
            _CACHE.clear()
            _CACHE["moe"] = synth.make_inputs(cfg, seed=0, B=B)
        return _CACHE["moe"]
    if "dense" not in _CACHE:
        _CACHE.clear()
        _CACHE["dense"] = synth.make_inputs(synth.B1, seed=0)
    base = _CACHE["dense"]
    if cfg == synth.B1:
        return base
    return dataclasses.replace(base, cfg=cfg, X=synth.make_x(cfg, seed=0, B=B))


def test_rankmixer_1b_full_size_256_samples(monkeypatch):
    """RankMixer-1B at B = 2048: prepared weights (the benchmark's launch), the same with the
    256 x 192 and four-wave 256 x 384 tiles forced, and row-major weights give the same
    bits; 256 samples (32 in each of the 8 row tiles) against the oracle, on X_L and on the
    pooled output."""
    cfg = synth.B1
    inp = _inputs(cfg)
    print(f"case 1B B={cfg.B} prepared weights", flush=True)
    o_pk, xl_pk = run_gpu(cfg, inp, packed=True)
    for policy in ("pair", "always"):
        print(f"case 1B B={cfg.B} prepared weights, RMX_WIDE_TILES={policy}", flush=True)
        monkeypatch.setenv("RMX_WIDE_TILES", policy)
        o_f, xl_f = run_gpu(cfg, inp, packed=True)
        monkeypatch.delenv("RMX_WIDE_TILES")
        assert np.array_equal(o_pk, o_f) and np.array_equal(xl_pk, xl_f), policy
    print(f"case 1B B={cfg.B} row-major weights", flush=True)
    o_rm, xl_rm = run_gpu(cfg, inp)
    assert np.array_equal(o_pk, o_rm) and np.array_equal(xl_pk, xl_rm)
    rows = sample_tiles(cfg.B, 32, seed=1)
    assert len(rows) == 256
    o_ref, xl_ref = run_oracle(cfg, inp, rows)
    check(cfg, o_pk[rows], xl_pk[rows], o_ref, xl_ref, f"1B B=2048 ({len(rows)} samples)")


@pytest.mark.parametrize("B", [64, 256, 1024, 4096])
def test_rankmixer_1b_serving_sweep(B):
    """The serving sweep (10 % of token rows zeroed) at its batch sizes, with the tile
    shapes the launch picks there (64-row tiles at 64; one round of 128 x 384 tiles for
    GEMM2 at 256; 256 x 384 tiles above), prepared and row-major weights bit-identical."""
    cfg = synth.SWEEP.with_(B=B)
    inp = _inputs(cfg, B)
    print(f"case 1B sweep B={B}", flush=True)
    o_pk, xl_pk = run_gpu(cfg, inp, packed=True)
    o_rm, xl_rm = run_gpu(cfg, inp)
    assert np.array_equal(o_pk, o_rm) and np.array_equal(xl_pk, xl_rm)
    rows = sample_tiles(B, max(4, 64 // max(1, B // 256)), seed=B)
    o_ref, xl_ref = run_oracle(cfg, inp, rows)
    check(cfg, o_pk[rows], xl_pk[rows], o_ref, xl_ref, f"1B sweep B={B} ({len(rows)} samples)")


def test_rankmixer_1b_sweep_16384():
    """The largest serving batch: 64 samples across the 64 row tiles, pooled output only
    (X_L at this size is not kept)."""
    cfg = synth.SWEEP.with_(B=16384)
    inp = _inputs(cfg, 16384)
    print("case 1B sweep B=16384", flush=True)
    o, _ = run_gpu(cfg, inp, with_xl=False, packed=True)
    rows = sample_tiles(cfg.B, 1, seed=5)[::2]
    o_ref, xl_ref = run_oracle(cfg, inp, rows)
    check(cfg, o[rows], None, o_ref, None, f"1B sweep B=16384 ({len(rows)} samples)")


def _run_moe_lists(cfg, inp, packed):
    import rankmixer_block_forward_amd as rmx
    X, w = rmx.upload(inp)
    B = X.shape[0]
    with rmx.Handle.for_config(cfg, max_batch=B) as h:
        if packed:
            w["packed"] = h.pack_weights(w)
            w["We1"] = w["We2"] = None
        xl = torch.full_like(X, float("nan"))
        gates = torch.full((cfg.L, B, cfg.T, cfg.E), float("nan"), dtype=torch.float32, device="cuda")
        out, lists = h.forward_moe_lists(X, w, xl_out=xl, gate_out=gates)
        torch.cuda.synchronize()
        lists = {k: v.cpu().numpy() for k, v in lists.items()}
    return to_np(out), to_np(xl), to_np(gates), lists


def _check_gates_vs_oracle(g, g_ref, label):
    g_ref = np.stack(g_ref, axis=0)
    err = np.linalg.norm(g - g_ref) / max(np.linalg.norm(g_ref), 1e-30)
    assert err <= 1e-2, f"{label}: gate rel-L2 {err}"
    flip = (g > 0) != (g_ref > 0)
    assert np.all(np.abs(g_ref[flip]) < 2e-2), f"{label}: activity differs away from zero"
    # where the oracle's gate is clearly away from zero, the GPU's list membership agrees
    firm = np.abs(g_ref) > 2e-2
    assert np.array_equal((g > 0)[firm], (g_ref > 0)[firm]), label
    print(f"{label}: gate rel-L2 {err:.2e}, {int(flip.sum())} of {flip.size} near-zero gates differ in sign",
          flush=True)


@pytest.mark.parametrize("B,T,D,E,h,L", [(100, 4, 64, 4, 64, 2), (300, 2, 256, 8, 96, 1), (1, 4, 64, 2, 32, 1),
                                         (257, 8, 128, 3, 128, 2), (700, 2, 384, 8, 1152, 1),
                                         # D / T = 8 and one 8-column chunk per lane in the combine
                                         (60, 16, 128, 2, 32, 2),
                                         # the most experts a token may have
                                         (130, 4, 64, 16, 32, 2)])
def test_moe_routing_lists_bit_exact(B, T, D, E, h, L):
    cfg = synth.Config("moe", B=B, T=T, D=D, k=2, L=L, dtype="bf16", E=E, moe_hidden=h, bias_std=0.02)
    inp = synth.make_inputs(cfg, seed=B + E)
    packed = D % 384 == 0 and h % 384 == 0
    o, xl, g, lists = _run_moe_lists(cfg, inp, packed)
    frac = check_moe_lists(lists, g)
    o_ref, xl_ref, g_ref = oracle.forward(inp.X, inp.layers(), cfg.eps)
    check(cfg, o, xl, o_ref, xl_ref, f"moe lists {B}x{T}x{D} E{E} h{h} L{L} (active {frac})")
    _check_gates_vs_oracle(g, g_ref, f"moe lists {B}x{T}x{D} E{E}")


def test_rankmixer_1b_moe_full_size_lists_and_64_samples():
    """Sparse-MoE 1B at B = 2048: the routing lists of both blocks bit for bit; prepared
    and row-major expert weights give the same bits; 64 samples (8 per row tile of the
    batch) against the oracle on X_L and the pooled output."""
    cfg = synth.MOE
    inp = _inputs(cfg)
    print("case 1B MoE prepared expert weights", flush=True)
    o_pk, xl_pk, g_pk, lists = _run_moe_lists(cfg, inp, packed=True)
    frac = check_moe_lists(lists, g_pk)
    print(f"1B MoE routing lists bit-exact; active fraction per block {frac}", flush=True)
    print("case 1B MoE row-major expert weights", flush=True)
    o_rm, xl_rm, g_rm, lists_rm = _run_moe_lists(cfg, inp, packed=False)
    assert np.array_equal(g_pk, g_rm) and np.array_equal(o_pk, o_rm) and np.array_equal(xl_pk, xl_rm)
    for name in ("group_start", "tile_start"):
        assert np.array_equal(lists[name], lists_rm[name])
    rows = sample_tiles(cfg.B, 8, seed=3)
    sub = synth.Inputs(cfg, inp.X[rows], inp.W1, inp.b1, inp.W2, inp.b2, inp.ln1_g, inp.ln1_b,
                       inp.ln2_g, inp.ln2_b, inp.moe)
    o_ref, xl_ref, g_ref = oracle.forward(sub.X, sub.layers(), cfg.eps)
    check(cfg, o_pk[rows], xl_pk[rows], o_ref, xl_ref, f"1B MoE B=2048 ({len(rows)} samples)")
    _check_gates_vs_oracle(g_pk[:, rows], g_ref, "1B MoE B=2048")
