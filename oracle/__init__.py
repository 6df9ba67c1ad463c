"""CPU oracle of the MoE block forward.  Test infrastructure only: imported by
``tests/``, the smoke check and the CPU-baseline leg of the benchmark, never by
the product library."""
from .moe_oracle import (combine, expert_mlp, experts, forward, forward_tokens,
                         gather_rows, permute, route, router_logits, silu,
                         softmax_all, topk_ids)

__all__ = ["combine", "expert_mlp", "experts", "forward", "forward_tokens",
           "gather_rows", "permute", "route", "router_logits", "silu",
           "softmax_all", "topk_ids"]
