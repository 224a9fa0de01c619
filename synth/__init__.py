"""Seeded synthetic inputs for the MoE-layer hot path.

This package is shared by the fp64 oracle and the HIP path's tests and bench. It
holds workload shapes and random-number plumbing only: none of the layer's own
arithmetic (scoring, selection, capacity, layout, FFN, combine) lives here.
"""
from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
from .gen import make_inputs, make_expert_weights, sub_seed  # noqa: F401
