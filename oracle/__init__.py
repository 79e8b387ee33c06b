"""CPU oracle for the MoE-LoRA expert layer (test infrastructure only).

Only tests/, the smoke check and the bench's CPU-baseline leg may use this
package. It shares no code with the HIP library and imports nothing from it.
"""
from . import moe_oracle, accounting  # noqa: F401
from .moe_oracle import (ROUTERS, route, route_backward, permute, gather_rows,  # noqa: F401
                         expert_forward, expert_backward, combine, combine_backward,
                         layer_forward, layer_backward, merged_forward, merge_lora,
                         layer_forward_backward, router_logits, router_input_grad,
                         layer_with_router_and_shared)
