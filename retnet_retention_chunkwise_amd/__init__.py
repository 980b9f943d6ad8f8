"""libretention: multi-scale retention on AMD Instinct MI355X (gfx950).

The compute lives in hand-written HIP kernels behind a C ABI
(include/libretention.h); this package is the thin Python binding:

    chunkwise_fwd(q, k, v, gamma, C, state_in=None, state_out=True) -> (y, state_out)
    chunkwise_fwd_noalloc(q, k, v, gamma, C, state_in=None, state_out=None, y=None) -> y
        (the same with no allocation inside the call: static device scratch)
    chunkwise_bwd(q, k, v, gamma, C, grad_y, state_in=None, grad_state_out=None)
        -> (grad_q, grad_k, grad_v, grad_state_in)
    parallel_fwd(q, k, v, gamma, state_in=None) -> y
    recurrent_step(q, k, v, gamma, state) -> y          (state updated in place)
    group_norm(y, weight=None, bias=None, eps=1e-5) -> out   (per-head GroupNorm of y)
    chunkwise_fwd_group_norm(q, k, v, gamma, C, weight=None, bias=None, eps=1e-5, ...)
        -> (y, state_out)     (the forward with the GroupNorm fused into its stores)
    fused_group_norm_failed(workspace, B, H, T, dk, dv, C, dtype) -> bool
        (whether a wait of that fused call gave up; its error word)

Build the library with ``python -m retnet_retention_chunkwise_amd.build``.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    MAX_CHUNK,
    MAX_DK,
    MAX_DV,
    RetentionError,
    chunkwise_bwd,
    chunkwise_fwd,
    chunkwise_fwd_group_norm,
    chunkwise_fwd_noalloc,
    chunkwise_workspace_bytes,
    fused_group_norm_failed,
    group_norm,
    last_error,
    load,
    parallel_fwd,
    recurrent_step,
    testing_gn_wait,
    version,
)
