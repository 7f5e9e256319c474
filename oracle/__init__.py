"""CPU oracle of the MoE layer (test infrastructure only; see oracle/moe.py)."""
from .moe import (capacity, combine, dispatch, effective_capacity, expert_ffn,
                  expert_ffn_streamed, expert_stats, gate_weights, moe_layer, permute,
                  router_logits, routing_record, select_topk, selection_logits, silu,
                  swiglu_ffn, token_outputs)

__all__ = ["capacity", "combine", "dispatch", "effective_capacity", "expert_ffn",
           "expert_ffn_streamed", "expert_stats", "gate_weights", "moe_layer", "permute",
           "router_logits", "routing_record", "select_topk", "selection_logits", "silu",
           "swiglu_ffn", "token_outputs"]
