"""fp64 CPU oracle of the RankMixer block forward and backward (test infrastructure only).

Imported only by the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline; the GPU library never imports it and shares no code with it.
"""
from .rmx_oracle import (tokenize, token_mix, layer_norm, gelu, pffn, moe_gates, moe_pffn,  # noqa: F401
                         self_attention, block, forward)
from .rmx_backward import (gelu_grad, layer_norm_backward, token_mix_backward,  # noqa: F401
                           pffn_backward, block_backward, backward, bce_logit_head)
from .rmx_mxfp8 import e4m3_round, mx_scale_exponent, mx_qdq, quantize_weights, forward_mxfp8  # noqa: F401
