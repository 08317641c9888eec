"""The no-allocation forward (rmx_block_forward_noalloc) through the C ABI: its output
equals the handle forward's (rmx_block_forward) bit for bit on the same inputs, on two calls
in a row whose second takes a smaller batch (the fixed workspace keeps the first call's
contents), for prepared and row-major weights; sizes beyond the fixed workspace are
refused on the host; and the calls take no device memory (free device memory unchanged
across them)."""
import ctypes

import numpy as np
import pytest

from rankmixer_block_forward_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _handle_forward(cfg, X, w):
    import rankmixer_block_forward_amd as rmx
    with rmx.Handle.for_config(cfg, max_batch=X.shape[0]) as h:
        out = h.forward(X, w)
        torch.cuda.synchronize()
    return out


def _free_bytes():
    free, total = torch.cuda.mem_get_info()
    return free


@pytest.mark.parametrize("cfg,batches", [
    (synth.Config("na-bf16", B=300, T=4, D=384, k=4, L=2, bias_std=0.02), (300, 57)),
    (synth.Config("na-fp32", B=70, T=4, D=64, k=2, L=2, dtype="fp32", bias_std=0.05), (70, 9)),
    (synth.SWEEP.with_(B=256), (256, 64)),
])
@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_matches_handle_forward_on_two_calls(cfg, batches, packed):
    import rankmixer_block_forward_amd as rmx
    if packed and cfg.dtype != "bf16":
        pytest.skip("prepared weights are bf16")
    print(f"case {cfg.name} packed={packed} batches={batches}", flush=True)
    inp = synth.make_inputs(cfg, seed=31, B=max(batches))
    X, w = rmx.upload(inp)
    if packed:
        with rmx.Handle.for_config(cfg, max_batch=1) as h:
            wp = dict(w, packed=h.pack_weights(w))
        del wp["W1"], wp["W2"]
    else:
        wp = w
    # want: the handle forward of each batch; got: two no-allocation calls in a row
    want = [_handle_forward(cfg, X[:B].contiguous(), wp) for B in batches]
    outs = [torch.full((B, cfg.D), float("nan"), dtype=torch.float32, device="cuda") for B in batches]
    Xs = [X[:B].contiguous() for B in batches]
    torch.cuda.synchronize()
    rmx.forward_noalloc(Xs[0], wp, cfg.T, cfg.D, cfg.k, cfg.L, cfg.dtype, cfg.eps, out=outs[0])  # sets the device up
    torch.cuda.synchronize()
    free0 = _free_bytes()
    rmx.forward_noalloc(Xs[1], wp, cfg.T, cfg.D, cfg.k, cfg.L, cfg.dtype, cfg.eps, out=outs[1])
    rmx.forward_noalloc(Xs[0], wp, cfg.T, cfg.D, cfg.k, cfg.L, cfg.dtype, cfg.eps, out=outs[0])
    rmx.forward_noalloc(Xs[1], wp, cfg.T, cfg.D, cfg.k, cfg.L, cfg.dtype, cfg.eps, out=outs[1])
    torch.cuda.synchronize()
    assert _free_bytes() == free0
    for B, o, ref in zip(batches, outs, want):
        assert torch.equal(o, ref), f"{cfg.name} B={B} packed={packed}"


def test_noalloc_refuses_what_it_cannot_hold():
    import rankmixer_block_forward_amd as rmx
    from rankmixer_block_forward_amd import binding
    lib = rmx.load_library()
    cfg = synth.B1
    X = torch.zeros((257, cfg.T, cfg.D), dtype=torch.bfloat16, device="cuda")
    w = {n: torch.zeros(1, dtype=torch.bfloat16, device="cuda") for n in ("W1", "W2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")}
    out = torch.full((257, cfg.D), 5.0, device="cuda")
    with pytest.raises(binding.RmxError) as e:
        rmx.forward_noalloc(X, w, cfg.T, cfg.D, cfg.k, cfg.L, out=out)   # 257 samples exceed the workspace
    assert e.value.status == binding.RMX_ERR_UNSUPPORTED and "limit" in str(e.value)
    moe = binding.rmx_config(4, 64, 2, 1, binding.RMX_BF16, 1e-5, 8, 2, 64, binding.RMX_ROUTING_MIX)
    st = lib.rmx_block_forward_noalloc(ctypes.byref(moe), None, 8, None, None, None)
    assert st == binding.RMX_ERR_UNSUPPORTED
    # X in host memory: refused on the host, nothing enqueued
    small = binding.rmx_config(4, 64, 2, 1, binding.RMX_BF16, 1e-5, 4, 0, 0, binding.RMX_ROUTING_MIX)
    host = np.zeros(4 * 4 * 64, dtype=np.uint16)
    out_small = torch.full((4, 64), 5.0, device="cuda")
    ws = binding._weights_struct(w, torch.bfloat16)
    st = lib.rmx_block_forward_noalloc(ctypes.byref(small), host.ctypes.data_as(ctypes.c_void_p), 4, ctypes.byref(ws),
                                       ctypes.c_void_p(out_small.data_ptr()), None)
    assert st == binding.RMX_ERR_INVALID_ARG and "X" in lib.rmx_last_error(None).decode()
    torch.cuda.synchronize()
    assert torch.all(out == 5.0) and torch.all(out_small == 5.0)
