"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

Holds only random draws and memory layouts, none of the method's arithmetic.
"""
from .configs import CONFIGS, StepConfig, by_index, small  # noqa: F401
from .inputs import StepInputs, f32_to_bf16_bits  # noqa: F401
