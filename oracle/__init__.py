"""CPU oracle of the MoE layer forward (test infrastructure only).

Only the tests, the entry module's smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.
"""
from .moe_oracle import (  # noqa: F401
    brute_forward, capacity, combine_from_experts, combine_rows, dispatch, drop_rate, expert_counts,
    expert_hidden, expert_mlp, expert_order, expert_output, fallback_choices, padded, reroute, f64, gate_values, gelu_erf, imbalance, moe_forward, relu,
    route, router_logits, router_stats, select_topk, silu, softmax, switch_aux_loss, topk_margin, with_shared,
)
