"""CPU oracle for the sparse MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Plain NumPy, fp64 (fp32 only where a page fixes it).  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does, and shares no code with it.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (ExpertBank, as_f64, bf16_to_f64, bias_update,  # noqa: F401
                         capacity_for, combine, dequant_u4_affine, dispatch,
                         expert_forward, ffn_and_combine,
                         group_select_from_logits, group_selection_scores,
                         layer, layer_stats, near_tie_flags, rank_descending,
                         route, route_from_logits, router_logits,
                         select_from_logits, sigmoid_f32, silu, softmax)
