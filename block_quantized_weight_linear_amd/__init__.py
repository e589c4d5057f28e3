"""MI355X (gfx950) Q8_0 block-quantized weight linear.

Python binding of the C ABI in include/q8_linear.h (and the measurement aids of
include/q8_probe.h) (libq8linear.so, built in-tree by
``python -m block_quantized_weight_linear_amd.build``).  PyTorch provides device
memory and streams; all computation runs in the library's HIP kernels.
"""

from ._binding import (  # noqa: F401
    LIB_PATH,
    Q8Error,
    abi_version,
    lib,
    moe_route_topk,
    probe_empty,
    probe_shape_count,
    probe_stream_read,
    q4_0_linear,
    q4_0_linear_fused_gate_up_silu,
    q4_k_linear,
    q4_k_linear_fused_gate_up_silu,
    q5_k_linear,
    q5_k_linear_fused_gate_up_silu,
    q6_k_linear,
    q6_k_linear_fused_gate_up_silu,
    moe_route_workspace_bytes,
    q8_linear,
    q8_linear_fused_gate_up_silu,
    q8_linear_fused_gate_up_silu_q8act,
    q8_linear_q8act,
    q8_moe_grouped_linear,
    q8_moe_grouped_linear_noalloc,
    q8_moe_workspace_bytes,
    q8_quantize_act,
)
