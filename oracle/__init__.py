"""CPU oracle of the routed MoE SwiGLU layer (test infrastructure only).

Only tests, the smoke check and the bench's CPU-baseline leg may import this
package.  The product library never does.
"""
from .moe_oracle import (  # noqa: F401
    backward, capacity, dequantize, dsilu, expert_choice_backward, expert_choice_capacity, expert_choice_forward,
    expert_choice_routing, expert_choice_weights_backward,
    e2m1_decode, e2m1_encode, e4m3_encode, expert_ffn, expert_ffn_backward, forward, fp8_e4m3fn_decode, logit_error_bound, mx4_dequantize, mx4_quantize, mx_dequantize, mx_quantize, mx_roundtrip,
    permute,
    router_logits, router_telemetry, routing_certificate, routing_weights, routing_weights_backward, silu,
    softmax_rows, topk_select,
)
