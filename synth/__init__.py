"""Seeded synthetic inputs for the ReplaySSM decode path.

This package is shared by the fp64 oracle (``oracle/``) and the HIP path
(``attention_decode_mamba_amd``).  It holds only the *input recipe* (shapes,
distributions, seeds, dtype casts) and none of the method's arithmetic: no
state update, no decay products, no replay or fold.
"""
from .workloads import WORKLOADS, Workload, get_workload
from .gen import (
    bf16_bits_from_f32,
    head_params,
    initial_state,
    decode_inputs,
    draft_inputs,
    accept_counts, draft_tree,
    special_decode_inputs, special_draft_inputs,
    stack_decode_inputs,
    stack_draft_inputs,
)

__all__ = [
    "WORKLOADS", "Workload", "get_workload",
    "bf16_bits_from_f32", "head_params", "initial_state",
    "decode_inputs", "draft_inputs", "accept_counts", "draft_tree",
    "special_decode_inputs", "special_draft_inputs",
    "stack_decode_inputs", "stack_draft_inputs",
]
