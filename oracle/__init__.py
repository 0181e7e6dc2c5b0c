"""CPU oracle for the routed-MoE forward (test infrastructure only)."""
from .moe_oracle import (RouteCfg, accumulate_load, combine, dequantize_mxfp4,  # noqa: F401
                         dequantize_rows, e2m1_decode, e8m0_decode, expert_mlp, forward, forward_tokens, fp8_e4m3_decode, gelu, gelu_tanh,
                         glu, group_scores,
                         keys_are_raw_logits, map_to_physical, permute, rmsnorm, route,
                         route_weights, router_logits, run_experts, score, select_experts,
                         selection_keys, shared_expert, silu, softplus)
