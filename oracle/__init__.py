"""CPU float64 oracle for the Q8_0 block-quantized linear.

Test infrastructure: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the HIP
library.
"""

from .q8_oracle import (  # noqa: F401
    ACT_ZERO_BELOW,
    QK8_0,
    Q8_0_BLOCK_BYTES,
    bf16_round_ref,
    Q4_0_BLOCK_BYTES,
    QK4_0,
    dequantize_q4_0,
    dequantize_q8_0,
    fused_gate_up_silu_q4_0_ref,
    fused_gate_up_silu_codes_ref,
    fused_gate_up_silu_q8act_ref,
    fused_gate_up_silu_ref,
    moe_mixture_ref,
    moe_ref,
    parse_q4_0,
    parse_q8_0,
    q4_0_linear_ref,
    q4_0_row_bytes,
    quantize_act_q8_ref,
    q8_0_row_bytes,
    q8_linear_bf16_operands_ref,
    q8_linear_codes_ref,
    q8_linear_q8act_ref,
    q8_linear_ref,
    rel_err_row_max,
    rel_err_row_norm,
    route_topk_p_ref,
    route_topk_ref,
    router_logits_ref,
    sigmoid_ref,
    silu_ref,
    softmax_ref,
)
