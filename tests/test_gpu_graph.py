"""The forward inside a captured HIP graph (torch.cuda.CUDAGraph over the caller's stream).

rmx_block_forward allocates nothing, synchronises nothing and enqueues only kernel launches
(no memset or copy nodes), so a caller may capture it once and replay it.  Each replay must
give the eager call's bits; between replays the test runs eager work of its own and
synchronises (replays of a graph whose nodes were wrongly recorded show up only from the
second replay on), and it changes the input in place to show that a replay reads the live
buffers, as the eager call would.
"""
import numpy as np
import pytest

from rankmixer_block_forward_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    (synth.Config("graph-bf16", B=300, T=4, D=384, k=4, L=2, bias_std=0.02), False),
    (synth.Config("graph-bf16-pk", B=300, T=4, D=384, k=4, L=2, bias_std=0.02), True),
    (synth.TINY, False),
]


@pytest.mark.parametrize("cfg,packed", CASES, ids=[c[0].name for c in CASES])
def test_forward_replays_from_a_captured_graph(cfg, packed):
    import rankmixer_block_forward_amd as rmx
    inp = synth.make_inputs(cfg, seed=31)
    inp2 = synth.make_inputs(cfg, seed=32)
    X, w = rmx.upload(inp)
    X2, _ = rmx.upload(inp2)
    with rmx.Handle.for_config(cfg, max_batch=X.shape[0]) as h:
        if packed:
            w = dict(w, packed=h.pack_weights(w))
            del w["W1"], w["W2"]
        ref = h.forward(X, w)
        ref2 = h.forward(X2, w)
        torch.cuda.synchronize()
        out = torch.full_like(ref, float("nan"))
        Xg = X.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):          # one eager call on the capturing stream first
            h.forward(Xg, w, out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            h.forward(Xg, w, out=out)
        for rep in range(3):
            out.fill_(float("nan"))            # eager work between the replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"replay {rep}"
        Xg.copy_(X2)                           # the replay reads the live input
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref2)
        assert not np.array_equal(ref.cpu().numpy(), ref2.cpu().numpy())
