"""FP64 CPU oracle of the routed MoE layer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The product path never does.
"""
from .moe_oracle import (  # noqa: F401
    backward,
    bf16_to_f64,
    brute_force_forward,
    combine,
    e4m3_to_f64,
    e8m0_to_f64,
    expert_lora_rank,
    expert_weight_grads,
    f64_to_bf16_bits,
    forward,
    lora_delta,
    mx_to_f64,
    permute_routes,
    route_gates,
    routed_rows,
    router_logits,
    select_routes,
    shared_expert,
    shared_expert_grads,
    sigmoid,
    silu,
    swiglu_expert,
)
from .moe_oracle import _swiglu_backward as swiglu_backward  # noqa: F401
