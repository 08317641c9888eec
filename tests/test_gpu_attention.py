"""GPU parity of the self-attention routing comparator (routing = RMX_ROUTING_ATTENTION)
against the fp64 oracle, through the C ABI.  Same bars as the forward: fp32 rel-L2 <= 1e-5;
bf16 rel-L2 <= 1e-2 and max-abs <= 5e-2 on X_L and on out (Q, K, V are stored in bf16 like
S and H; scores, softmax and the weighted sum are fp32)."""
import numpy as np
import pytest

from rankmixer_block_forward_amd import synth
from tests.parity import check, run_gpu, run_oracle, sample_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    # the scalar row path with generic products; bf16 with ragged rows and biases; the 100M
    # shape (T = 16, D = 768) at a ragged batch; the largest T the softmax takes (one key per
    # lane); a single sample
    synth.TINY.with_(name="attn-tiny-fp32", routing="attention"),
    synth.Config("attn-fp32-vec", B=6, T=4, D=64, k=2, L=2, dtype="fp32", bias_std=0.1, routing="attention"),
    synth.Config("attn-bf16-48", B=48, T=4, D=256, k=4, L=2, bias_std=0.05, routing="attention"),
    synth.Config("attn-100m-300", B=300, T=16, D=768, k=4, L=2, routing="attention"),
    synth.Config("attn-t64", B=20, T=64, D=512, k=2, L=2, routing="attention"),
    synth.Config("attn-one", B=1, T=8, D=256, k=4, L=1, routing="attention"),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_attention_routing_matches_oracle(cfg):
    print(f"case {cfg.name}", flush=True)
    inp = synth.make_inputs(cfg, seed=31)
    o, xl = run_gpu(cfg, inp)
    o_ref, xl_ref = run_oracle(cfg, inp)
    check(cfg, o, xl, o_ref, xl_ref, cfg.name)


@pytest.mark.slow
def test_attention_routing_1b_full_size_sampled_rows():
    """The 1B shape (T = 32, D = 1536) at B = 2048 with attention routing; the oracle on 6
    sampled samples."""
    cfg = synth.B1_ATTN
    inp = synth.make_inputs(cfg, seed=0)
    o, xl = run_gpu(cfg, inp)
    rows = sample_rows(cfg.B, 6, seed=32)
    o_ref, xl_ref = run_oracle(cfg, inp, rows)
    check(cfg, o[rows], xl[rows], o_ref, xl_ref, "1B attention, sampled rows")


def test_attention_routing_argument_errors():
    import rankmixer_block_forward_amd as rmx
    from rankmixer_block_forward_amd.binding import RmxError, RMX_ERR_UNSUPPORTED, RMX_ERR_INVALID_ARG
    cfg = CASES[2]
    inp = synth.make_inputs(cfg, seed=33)
    X, w = rmx.upload(inp)
    with rmx.Handle.for_config(cfg) as h:
        with pytest.raises(RmxError) as ei:        # prepared weights: Token Mixing path only
            h.forward(X, dict(w, packed=h.pack_weights(w)))
        assert ei.value.status == RMX_ERR_UNSUPPORTED
        with pytest.raises(RmxError) as ei:        # no training for the comparator
            h.forward_train(X, w)
        assert ei.value.status == RMX_ERR_UNSUPPORTED
        with pytest.raises(RmxError) as ei:        # the projections are required
            h.forward(X, {k: v for k, v in w.items() if k != "Wk"})
        assert ei.value.status == RMX_ERR_INVALID_ARG
    mix = cfg.with_(routing="mix")
    with rmx.Handle.for_config(mix) as h:
        with pytest.raises(RmxError) as ei:        # projections given to a Token Mixing handle
            h.forward(X, w)
        assert ei.value.status == RMX_ERR_INVALID_ARG
    torch.cuda.synchronize()
