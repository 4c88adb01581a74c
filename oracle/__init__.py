"""fp64 CPU oracle for the MoE FFN layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the HIP library never does, and this package never touches it.
"""
from .moe_oracle import (capacity, combine, combine_weights, dispatch, expert_outputs, ffn,
                         gate_logits, gelu, layer_forward, layer_rows, max_rows, route, softmax,
                         top_k)

__all__ = ["capacity", "combine", "combine_weights", "dispatch", "expert_outputs", "ffn",
           "gate_logits", "gelu", "layer_forward", "layer_rows", "max_rows", "route", "softmax",
           "top_k"]
