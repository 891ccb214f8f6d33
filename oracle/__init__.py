"""CPU oracle for the LongCat-Flash zero-computation-expert MoE layer.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously-correct
reference that the HIP path is checked against. Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never does, and the two share no code.

Source of what is computed: "LongCat-Flash" (llm-wiki entity page), section
2.1 "Zero-Computation Experts" (the MoE sum, the zero-expert identity, the
expert-bias update and its symbols, and the device-level load-balance loss
with the zero experts as one extra group), section 2.3.2 (softmax gating), the
training-stability section (hidden z-loss), and the model table in section 1
"核心参数" (layer shape).
"""

from .lcmoe_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    e4m3fn_value_table,
    dequant_fp8_blocks,
    e4m3fn_encode,
    quantize_rows_fp8,
    dequant_rows_fp8,
    round_to_bf16,
    expert_ffn_a8,
    expert_gate_up,
    expert_down_fp8_rows,
    router_logits,
    selection_scores,
    select_topk,
    softmax_gates,
    expert_counts,
    permutation,
    silu,
    expert_ffn,
    combine_given_routing,
    combine_given_expert_outputs,
    route,
    forward,
    dense_masked_forward,
    bias_update,
    expert_groups,
    load_balance_stats,
    hidden_z_loss,
    silu_grad,
    expert_backward,
    layer_backward,
)
