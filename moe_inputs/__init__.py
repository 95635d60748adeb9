"""Seeded synthetic inputs and workload shapes for the MoE layer (no method arithmetic)."""

from .configs import ORDER, WORKLOADS, MoEConfig, small_case  # noqa: F401
from .gen import (  # noqa: F401
    Bf16, as_f32, bf16_bits_rne, bf16_bits_to_f32, generate, generate_bypass, generate_dy,
    relu_logit_offset)
