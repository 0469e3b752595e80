"""MI355X-native SALR linear layer.

SALR (Sparsity-Aware Low-Rank Representation) serves a linear layer as
Y = X W_s^T + (X A_cat) B_cat: W_s is the frozen weight after a static
per-row magnitude prune, stored as a bitmap plus packed bf16 values, and
A_cat / B_cat stack the truncated-SVD residual adapter with the LoRA
adapters.  Encode, forward and the adapter backward run in hand-written gfx950 HIP kernels behind
the C ABI of include/salr.h (libsalr.so); this package only marshals
arguments (binding.py) and draws synthetic inputs (synth.py).
"""

from .binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    NOALLOC_SCRATCH_BYTES,
    SalrError,
    SalrLayer,
    SalrMoE,
    WaitTimeout,
    backward_workspace,
    backward_ws_bytes,
    encode,
    forward_workspace,
    fuse,
    lib,
    linear_backward,
    linear_forward,
    linear_forward_noalloc,
    moe_encode_expert,
    moe_forward,
    moe_query_sizes,
    moe_workspace,
    nf4_levels,
    probe_mfma,
    probe_stream_read,
    quantize_nf4,
    query_sizes,
    transpose_count,
    transpose_layer,
    transpose_ws_bytes,
    wait_error,
    workspace,
)

__all__ = [
    "EXPORTS", "LIB_PATH", "NOALLOC_SCRATCH_BYTES", "SalrError", "SalrLayer", "SalrMoE", "WaitTimeout", "backward_workspace",
    "backward_ws_bytes", "encode", "forward_workspace", "fuse", "lib", "linear_backward", "linear_forward",
    "linear_forward_noalloc", "moe_encode_expert", "moe_forward", "moe_query_sizes", "moe_workspace", "nf4_levels", "probe_mfma", "probe_stream_read", "quantize_nf4", "query_sizes",
    "transpose_count", "transpose_layer", "transpose_ws_bytes", "wait_error", "workspace",
]
