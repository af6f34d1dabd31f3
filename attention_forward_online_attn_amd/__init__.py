"""MI355X (gfx950) fused attention forward: dense, causal, forward-mode JVP,
additive bias / boolean mask and jagged multi-head variants, and the dense
backward, behind the C ABI declared in include/attn.h.

The Python layer only marshals arguments: every step of the computation runs
in the HIP kernels of libattn_mi355x.so.  torch supplies device memory and the
current stream.
"""

from .binding import (  # noqa: F401
    AttnError,
    bwd,
    bwd_bias,
    bwd_workspace_bytes,
    fwd,
    fwd_bias,
    fwd_jvp,
    jagged_bwd,
    jagged_bwd_workspace_bytes,
    jagged_fwd,
    jagged_fwd_noalloc,
    jagged_workspace_bytes,
    library_path,
    load_library,
)
