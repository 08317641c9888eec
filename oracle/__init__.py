"""fp64 CPU oracle of the RankMixer block forward (test infrastructure only).

Imported only by the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline; the GPU library never imports it and shares no code with it.
"""
from .rmx_oracle import (tokenize, token_mix, layer_norm, gelu, pffn, moe_gates, moe_pffn,  # noqa: F401
                         block, forward)
