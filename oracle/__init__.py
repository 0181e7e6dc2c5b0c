"""CPU oracle for the routed-MoE forward (test infrastructure only)."""
from .moe_oracle import (RouteCfg, combine, expert_mlp, forward, forward_tokens,  # noqa: F401
                         group_scores, keys_are_raw_logits, permute, rmsnorm, route,
                         route_weights, router_logits, run_experts, score,
                         select_experts, selection_keys, shared_expert, silu, softplus)
