"""CPU float64 oracle of the gpt-oss MoE block forward (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use it."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (widen, router_logits, select_topk, routing_weights, route,  # noqa: F401
                         clamped_glu, expert_mlp, expert_permutation, moe_forward,
                         moe_forward_dense, near_ties, clamp_fraction, GLU_ALPHA, GLU_LIMIT)
