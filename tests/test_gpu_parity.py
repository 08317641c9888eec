"""Parity of the HIP path (through the C ABI) with the fp64 oracle on seeded inputs.

Small shapes are compared element by element in full; the full-size workloads
(RankMixer-100M at B=512, RankMixer-1B at B=2048, the serving sweep) run on the GPU at
their real size, in the launch configuration the benchmark times, and are compared on
sampled samples that the oracle computes one by one (samples are independent: mixing,
LayerNorm and the per-token FFN never cross samples).
"""
import ctypes

import numpy as np
import pytest

import oracle
from rankmixer_block_forward_amd import synth
from tests.parity import check, run_gpu, run_oracle, sample_rows, sample_tiles, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _rmx():
    import rankmixer_block_forward_amd as rmx
    return rmx


# ------------------------------------------------------------------ Token Mixing

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,T,D", [(3, 4, 8), (7, 4, 12), (5, 16, 768), (2, 32, 1536), (4, 2, 6), (1, 1, 16)])
def test_token_mix_bit_exact(dtype, B, T, D):
    rmx = _rmx()
    cfg = synth.Config("mix", B=B, T=T, D=D, k=1, L=1, dtype=dtype)
    X = synth.make_x(cfg, seed=B * 131 + D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Xd = torch.from_numpy(X).cuda().to(tdt)
    Y = rmx.token_mix(Xd)
    Z = rmx.token_mix(Y)
    torch.cuda.synchronize()
    want = oracle.token_mix(X.astype(np.float64))
    assert np.array_equal(to_np(Y).astype(np.float64), want)
    assert torch.equal(Z, Xd)  # H = T: the permutation is its own inverse


# ------------------------------------------------------------------------ fp32

def test_tiny_workload_fp32():
    cfg = synth.TINY
    inp = synth.make_inputs(cfg, seed=0)
    o, xl = run_gpu(cfg, inp)
    o_ref, xl_ref = run_oracle(cfg, inp)
    check(cfg, o, xl, o_ref, xl_ref, "tiny")


@pytest.mark.parametrize("B,T,D,k,L", [(37, 4, 64, 2, 2), (5, 3, 12, 3, 1), (130, 8, 128, 4, 2),
                                       (1, 2, 6, 1, 3), (65, 4, 8, 2, 1)])
def test_fp32_shapes(B, T, D, k, L):
    cfg = synth.Config("fp32", B=B, T=T, D=D, k=k, L=L, dtype="fp32", bias_std=0.05)
    inp = synth.make_inputs(cfg, seed=B + D)
    o, xl = run_gpu(cfg, inp)
    o_ref, xl_ref = run_oracle(cfg, inp)
    check(cfg, o, xl, o_ref, xl_ref, f"fp32 {B}x{T}x{D} k{k} L{L}")


def test_zero_token_rows_fp32():
    cfg = synth.TINY.with_(B=16, zero_frac=0.25, bias_std=0.1, ln_init="jitter")
    inp = synth.make_inputs(cfg, seed=3)
    o, xl = run_gpu(cfg, inp)
    o_ref, xl_ref = run_oracle(cfg, inp)
    check(cfg, o, xl, o_ref, xl_ref, "fp32 zero rows")


# ------------------------------------------------------------------------ bf16

@pytest.mark.parametrize("B,T,D,k,L", [
    (300, 4, 256, 4, 2),   # MFMA path: 2 M tiles (ragged), 4 N tiles in GEMM1
    (77, 5, 320, 2, 1),    # MFMA path, ragged N tiles (640 = 2.5 x 256, 320 = 1.25 x 256)
    (50, 4, 96, 2, 2),     # 64-row tiles, odd K-step count (K = 96)
    (50, 5, 40, 2, 2),     # K = 40 not a multiple of 32: generic kernel in bf16
    (1, 16, 768, 4, 2),    # one sample at the 100M width (64-row tiles)
    (64, 8, 512, 4, 1),    # one full 64-row tile
    (128, 8, 512, 4, 1),   # largest batch on the 64-row tiles
    (129, 8, 512, 4, 1),   # smallest batch on the 256-row tiles
    (513, 16, 768, 4, 1),  # one row past a tile boundary
])
def test_bf16_shapes(B, T, D, k, L):
    cfg = synth.Config("bf16", B=B, T=T, D=D, k=k, L=L, dtype="bf16", bias_std=0.02)
    inp = synth.make_inputs(cfg, seed=B + D + L)
    o, xl = run_gpu(cfg, inp)
    rows = sample_rows(B, 64)
    o_ref, xl_ref = run_oracle(cfg, inp, rows)
    check(cfg, o[rows], xl[rows], o_ref, xl_ref, f"bf16 {B}x{T}x{D} k{k} L{L}")


def test_bf16_zero_rows_and_biases():
    cfg = synth.Config("bf16z", B=200, T=8, D=128, k=4, L=2, dtype="bf16", bias_std=0.05, zero_frac=0.3)
    inp = synth.make_inputs(cfg, seed=9)
    o, xl = run_gpu(cfg, inp)
    o_ref, xl_ref = run_oracle(cfg, inp)
    check(cfg, o, xl, o_ref, xl_ref, "bf16 zero rows")


def test_bf16_deterministic():
    cfg = synth.Config("det", B=300, T=4, D=256, k=4, L=2, dtype="bf16")
    inp = synth.make_inputs(cfg, seed=1)
    o1, x1 = run_gpu(cfg, inp)
    o2, x2 = run_gpu(cfg, inp)
    assert np.array_equal(o1, o2) and np.array_equal(x1, x2)


# ------------------------------------------------------- full-size workloads

def test_small_batch_deterministic():
    """Few rows per token (64-row tiles): two runs agree bit for bit, and match the oracle."""
    cfg = synth.Config("small", B=33, T=8, D=256, k=4, L=2, dtype="bf16", bias_std=0.05)
    inp = synth.make_inputs(cfg, seed=21)
    o1, xl1 = run_gpu(cfg, inp)
    o2, xl2 = run_gpu(cfg, inp)
    assert np.array_equal(o1, o2) and np.array_equal(xl1, xl2)
    rows = sample_rows(cfg.B, 33)
    o_ref, xl_ref = run_oracle(cfg, inp, rows)
    check(cfg, o1[rows], xl1[rows], o_ref, xl_ref, "bf16 B=33")


@pytest.mark.parametrize("B,T,D,k,L", [
    (300, 4, 256, 4, 2),   # 256-row tiles, ragged rows
    (77, 5, 320, 2, 1),    # ragged column tiles (kD = 640, D = 320)
    (33, 8, 256, 4, 2),    # 64-row tiles
    (65, 8, 512, 4, 1),    # 64-row tiles, one row into the second
    (128, 8, 512, 4, 1),   # largest batch on the 64-row tiles
    (129, 8, 512, 4, 1),   # smallest batch on the 256-row tiles
    (1, 16, 768, 4, 2),    # one sample
    (300, 4, 384, 4, 2),   # 256 x 384 tiles in both products, ragged rows
    (129, 8, 384, 2, 1),   # 256 x 384 tiles, one row past the 64-row kernel
    (257, 4, 1152, 2, 1),  # 256 x 384 tiles, three (D) and six (kD) column tiles, two row tiles
    (300, 4, 256, 3, 2),   # GEMM1 on 256 x 384 tiles (kD = 768), GEMM2 on 256 x 256 (D = 256)
])
def test_prepared_weights_bit_identical(B, T, D, k, L, monkeypatch):
    """Weights prepared by rmx_pack_weights (and the packed S and H they bring) give the
    same bits as the row-major path, and match the oracle; the same with the 256 x 384 tiles
    (RMX_WIDE_TILES=always) or the 128 x 384 tiles (=half) forced where N % 384 == 0, the
    256 x 192 or 128 x 192 tiles two to a CU (=pair, =pairhalf) where N % 192 == 0, the
    256 x 384 tiles on eight waves (=wide8) where N % 384 == 0, with
    both forbidden (=never), and, up to 128 rows per token, with the 64 x 128 tiles forced
    or forbidden (RMX_NARROW_TILES), since at these sizes the launch picks by occupancy."""
    cfg = synth.Config("pk", B=B, T=T, D=D, k=k, L=L, dtype="bf16", bias_std=0.02)
    inp = synth.make_inputs(cfg, seed=B + 3 * D)
    o1, xl1 = run_gpu(cfg, inp)
    o2, xl2 = run_gpu(cfg, inp, packed=True)
    assert np.array_equal(o1, o2) and np.array_equal(xl1, xl2)
    for var, policy in (("RMX_WIDE_TILES", "always"), ("RMX_WIDE_TILES", "half"), ("RMX_WIDE_TILES", "pair"),
                        ("RMX_WIDE_TILES", "pairhalf"), ("RMX_WIDE_TILES", "wide8"), ("RMX_WIDE_TILES", "never"),
                        ("RMX_NARROW_TILES", "always"), ("RMX_NARROW_TILES", "never")):
        monkeypatch.setenv(var, policy)
        o3, xl3 = run_gpu(cfg, inp, packed=True)
        monkeypatch.delenv(var)
        assert np.array_equal(o1, o3) and np.array_equal(xl1, xl3), (var, policy)
    rows = sample_rows(B, 32)
    o_ref, xl_ref = run_oracle(cfg, inp, rows)
    check(cfg, o2[rows], xl2[rows], o_ref, xl_ref, f"prepared {B}x{T}x{D} k{k} L{L}")


def test_prepared_weights_rejected_where_unsupported():
    rmx = _rmx()
    from rankmixer_block_forward_amd import binding
    for cfg in (synth.TINY, synth.Config("moe", B=8, T=4, D=64, k=2, L=1, dtype="bf16", E=2, moe_hidden=64)):
        with rmx.Handle.for_config(cfg, max_batch=8) as h:
            assert h.packed_weights_bytes() == 0
            with pytest.raises(binding.RmxError):
                h.pack_weights({"W1": None, "W2": None})


def test_rankmixer_100m_full_size():
    cfg = synth.M100
    inp = synth.make_inputs(cfg, seed=0)
    o, xl = run_gpu(cfg, inp)
    o_pk, xl_pk = run_gpu(cfg, inp, packed=True)
    assert np.array_equal(o, o_pk) and np.array_equal(xl, xl_pk)
    rows = sample_tiles(cfg.B, 32)
    o_ref, xl_ref = run_oracle(cfg, inp, rows)
    check(cfg, o[rows], xl[rows], o_ref, xl_ref, f"100M B=512 ({len(rows)} samples)")


# ------------------------------------------------------------ boundary cases

def test_batch_zero_and_smaller_batches_reuse_handle():
    rmx = _rmx()
    cfg = synth.Config("reuse", B=40, T=4, D=64, k=2, L=2, dtype="bf16", bias_std=0.02)
    inp = synth.make_inputs(cfg, seed=5)
    X, w = rmx.upload(inp)
    with rmx.Handle.for_config(cfg, max_batch=64) as h:
        out0 = torch.empty((0, cfg.D), dtype=torch.float32, device="cuda")
        h.forward(X[:0], w, out=out0)  # B = 0: nothing enqueued
        for B in (40, 7, 1):
            out = h.forward(X[:B].contiguous(), w)
            torch.cuda.synchronize()
            o_ref, _ = oracle.forward(inp.X[:B], inp.layers(), cfg.eps)[:2]
            check(cfg, to_np(out), None, o_ref, None, f"reuse B={B}")


def test_errors_enqueue_nothing_and_leave_outputs_untouched():
    rmx = _rmx()
    cfg = synth.Config("err", B=8, T=4, D=64, k=2, L=1, dtype="bf16")
    inp = synth.make_inputs(cfg, seed=6)
    X, w = rmx.upload(inp)
    with rmx.Handle.for_config(cfg, max_batch=4) as h:
        out = torch.full((8, cfg.D), 7.0, device="cuda")
        with pytest.raises(rmx.RmxError) as e:
            h.forward(X, w, out=out)  # B = 8 > max_batch = 4
        assert e.value.status == 1
        with pytest.raises(rmx.RmxError):
            h.forward(X[:4].contiguous(), w, out=out[:4], L=2)  # L differs from the handle's
        with pytest.raises(rmx.RmxError):
            h.forward(X[:4].contiguous(), w, out=out[:4], k=4)
        # W1 in an allocation too small for T*D*kD elements (raw hipMalloc of half the bytes)
        hip = ctypes.CDLL("libamdhip64.so")
        half = ctypes.c_void_p()
        assert hip.hipMalloc(ctypes.byref(half), ctypes.c_size_t(w["W1"].numel())) == 0
        try:
            lib = rmx.load_library()
            ws = h._weights(w)
            ws.W1 = half.value
            st = lib.rmx_block_forward(h._h, ctypes.c_void_p(X.data_ptr()), 4, ctypes.byref(ws), 1, 2,
                                       ctypes.c_void_p(out.data_ptr()), None)
            assert st == 1 and "W1" in lib.rmx_last_error(h._h).decode()
        finally:
            hip.hipFree(half)
        # a host pointer is refused by the library itself
        lib = rmx.load_library()
        host = np.zeros(4 * 4 * 64, dtype=np.uint16)
        ws = h._weights(w)
        st = lib.rmx_block_forward(h._h, host.ctypes.data_as(ctypes.c_void_p), 4, ctypes.byref(ws), 1, 2,
                                   ctypes.c_void_p(out.data_ptr()), None)
        assert st == 1 and "X" in lib.rmx_last_error(h._h).decode()
        torch.cuda.synchronize()
        assert torch.all(out == 7.0)


def test_profile_counts_launches():
    rmx = _rmx()
    cfg = synth.Config("prof", B=64, T=4, D=64, k=2, L=2, dtype="bf16")
    inp = synth.make_inputs(cfg, seed=7)
    X, w = rmx.upload(inp)
    with rmx.Handle.for_config(cfg) as h:
        h.profile_enable(True)
        for _ in range(3):
            h.forward(X, w)
        p = h.profile_read()
        assert p["rows_ln2_mix_ln1"]["launches"] == 6
        assert p["gemm1_gelu"]["launches"] == 6 and p["gemm2_residual"]["launches"] == 6
        assert p["rows_ln2_pool"]["launches"] == 3 and p["_dropped"] == 0
        assert all(v["total_ms"] > 0 for k, v in p.items() if k != "_dropped")
        h.profile_reset()
        assert h.profile_read() == {"_dropped": 0}


# ------------------------------------------------------------------ Sparse-MoE

def _run_moe(cfg, inp, with_xl=True, packed=False):
    """The MoE forward; packed: on expert weights prepared by rmx_pack_weights (We1 and We2
    are then withheld, so the forward must read the prepared copy)."""
    rmx = _rmx()
    X, w = rmx.upload(inp)
    B = X.shape[0]
    with rmx.Handle.for_config(cfg, max_batch=B) as h:
        if packed:
            w["packed"] = h.pack_weights(w)
            w["We1"] = w["We2"] = None
        out = torch.full((B, cfg.D), float("nan"), dtype=torch.float32, device="cuda")
        xl = torch.full_like(X, float("nan")) if with_xl else None
        gates = torch.full((cfg.L, B, cfg.T, cfg.E), float("nan"), dtype=torch.float32, device="cuda")
        h.forward(X, w, out=out, xl_out=xl, gate_out=gates)
        torch.cuda.synchronize()
    return to_np(out), (to_np(xl) if with_xl else None), to_np(gates)


def _check_gates(g, g_ref, label):
    # gates come from the bf16 LN1 output on the GPU and from fp64 on the CPU: compare as
    # values (ReLU is continuous, so a sign flip near zero moves the output only by O(g))
    g_ref = np.stack(g_ref, axis=0)
    assert g.shape == g_ref.shape
    err = np.linalg.norm(g - g_ref) / max(np.linalg.norm(g_ref), 1e-30)
    assert err <= 1e-2, f"{label}: gate rel-L2 {err}"
    flip = (g > 0) != (g_ref > 0)
    assert np.all(np.abs(g_ref[flip]) < 2e-2), f"{label}: activity differs away from zero"
    print(f"{label}: gate rel-L2 {err:.2e}, active {float((g_ref > 0).mean()):.3f}", flush=True)


@pytest.mark.parametrize("B,T,D,E,h,L", [(100, 4, 64, 4, 64, 2), (300, 2, 256, 8, 96, 1), (1, 4, 64, 2, 32, 1),
                                         (257, 8, 128, 3, 128, 2)])
def test_moe_shapes(B, T, D, E, h, L):
    cfg = synth.Config("moe", B=B, T=T, D=D, k=2, L=L, dtype="bf16", E=E, moe_hidden=h, bias_std=0.02)
    inp = synth.make_inputs(cfg, seed=B + E)
    o, xl, g = _run_moe(cfg, inp)
    o_ref, xl_ref, g_ref = oracle.forward(inp.X, inp.layers(), cfg.eps)
    check(cfg, o, xl, o_ref, xl_ref, f"moe {B}x{T}x{D} E{E} h{h} L{L}")
    _check_gates(g, g_ref, f"moe {B}x{T}x{D} E{E}")


@pytest.mark.parametrize("B,T,D,E,h,L", [(100, 2, 384, 4, 384, 2), (300, 4, 384, 3, 768, 1), (1, 2, 768, 2, 384, 1),
                                         (700, 2, 384, 8, 1152, 1)])
def test_moe_prepared_weights_bit_identical(B, T, D, E, h, L):
    """Prepared expert weights (256 x 384 tiles, A rows gathered into the packed LDS layout)
    give the bits of the row-major expert products: same MFMA inputs in the same K order.
    Group row counts here are partial tiles, single tiles and several tiles with a tail."""
    cfg = synth.Config("moe-pk", B=B, T=T, D=D, k=2, L=L, dtype="bf16", E=E, moe_hidden=h, bias_std=0.02)
    inp = synth.make_inputs(cfg, seed=B + 7 * E)
    o1, xl1, g1 = _run_moe(cfg, inp)
    o2, xl2, g2 = _run_moe(cfg, inp, packed=True)
    assert np.array_equal(g1, g2)
    assert np.array_equal(o1, o2) and np.array_equal(xl1, xl2)
    rows = sample_rows(B, 16)
    sub = synth.Inputs(cfg, inp.X[rows], inp.W1, inp.b1, inp.W2, inp.b2, inp.ln1_g, inp.ln1_b,
                       inp.ln2_g, inp.ln2_b, inp.moe)
    o_ref, xl_ref, g_ref = oracle.forward(sub.X, sub.layers(), cfg.eps)
    check(cfg, o2[rows], xl2[rows], o_ref, xl_ref, f"moe prepared {B}x{T}x{D} E{E} h{h} L{L}")
    _check_gates(g2[:, rows], g_ref, f"moe prepared {B}x{T}x{D} E{E}")


def test_moe_prepared_weights_size_and_rejection():
    rmx = _rmx()
    from rankmixer_block_forward_amd import binding
    cfg = synth.Config("moe-pk", B=8, T=2, D=384, k=2, L=2, dtype="bf16", E=3, moe_hidden=384)
    with rmx.Handle.for_config(cfg, max_batch=8) as h:
        # per block and expert: We1^T (h = 384 rows of D) and We2^T (D = 384 rows of h), each
        # padded to 512 rows (whole 256-row blocks), bf16
        assert h.packed_weights_bytes() == 2 * 2 * 3 * (512 * 384 + 512 * 384) * 2
        X, w = rmx.upload(synth.make_inputs(cfg, seed=1))
        fake = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
        with pytest.raises(binding.RmxError):  # MXFP8 weights are a dense-only variant
            h.forward(X, dict(w, packed_mxfp8=fake))
    odd = synth.Config("moe-odd", B=8, T=2, D=384, k=2, L=1, dtype="bf16", E=2, moe_hidden=256)
    with rmx.Handle.for_config(odd, max_batch=8) as h:
        assert h.packed_weights_bytes() == 0
        X, w = rmx.upload(synth.make_inputs(odd, seed=1))
        with pytest.raises(binding.RmxError):
            h.pack_weights(w)
        fake = torch.empty(1 << 20, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(binding.RmxError):
            h.forward(X, dict(w, packed=fake))


def test_moe_zero_router_is_ffn_free_block():
    cfg = synth.Config("moe0", B=64, T=4, D=64, k=2, L=2, dtype="bf16", E=4, moe_hidden=64)
    inp = synth.make_inputs(cfg, seed=3)
    inp.moe["Wg"][:] = 0.0
    o, xl, g = _run_moe(cfg, inp)
    assert not g.any()
    o_ref, xl_ref, _ = oracle.forward(inp.X, inp.layers(), cfg.eps)
    check(cfg, o, xl, o_ref, xl_ref, "moe zero router")
