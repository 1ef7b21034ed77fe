"""CPU oracle for the MoE expert-layer forward pass -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (expert_layer_moe_amd) never does.
"""
from .moe_oracle import *  # noqa: F401,F403
