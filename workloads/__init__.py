"""Seeded synthetic inputs for the MoE FFN layer forward.

This package holds shapes, seeds and random draws only: no routing, no
expert math, no combine.  Both the CPU oracle (through the tests and the
benchmark's CPU leg) and the HIP path receive tensors produced here.
"""
from .configs import CONFIGS, MoeConfig, get_config, scaled_config
from .generate import generate, expert_slice

__all__ = ["CONFIGS", "MoeConfig", "get_config", "scaled_config", "generate", "expert_slice"]
