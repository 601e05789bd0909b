"""Gated DeltaNet-2 forward (chunked prefill and batched decode) for AMD
MI355X (gfx950): hand-written HIP kernels behind the C ABI of include/gdr2.h.

    from gated_delta_rule_86_amd import forward, decode_step
    o, S_final = forward(q, k, v, b, w, g, S0=None, chunk=64)
    o = decode_step(state, q, k, v, b, w, g)      # state updated in place

The HIP library is loaded on first use; importing this package does not
touch the GPU.
"""
from .gdr2 import Gdr2Error, decode_step, forward, load_library, workspace_size  # noqa: F401

__all__ = ["forward", "decode_step", "workspace_size", "load_library", "Gdr2Error"]
