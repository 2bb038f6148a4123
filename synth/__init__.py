"""Seeded synthetic inputs (no scan arithmetic); shared by the oracle's tests and the HIP path's tests and bench."""
from .inputs import WORKLOADS, Workload, bf16_bits, bf16_round, custom, make_block_inputs, make_inputs, make_mimo_proj, make_norm_params, make_state

__all__ = ["WORKLOADS", "Workload", "bf16_bits", "bf16_round", "custom", "make_block_inputs", "make_inputs", "make_mimo_proj", "make_norm_params", "make_state"]
