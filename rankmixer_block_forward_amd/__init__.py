"""RankMixer block forward on AMD MI355X (gfx950): HIP kernels behind a C ABI (librmx.so).

    from rankmixer_block_forward_amd import Handle, token_mix, tokenize
    h = Handle(T=32, D=1536, k=4, L=2, dtype="bf16", max_batch=2048)
    out = h.forward(X, weights)          # X [B, T, D] on the GPU -> out [B, D] fp32

The library is built in-tree with ``python -m rankmixer_block_forward_amd.build``.
"""
from .binding import (EXPORTS, Handle, RmxError, forward_noalloc, load_library, token_mix, tokenize,  # noqa: F401
                      upload)
