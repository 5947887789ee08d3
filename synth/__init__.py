"""Seeded synthetic inputs for the Medusa decode step.

This package only draws random tensors, rounds them to the storage dtype and
applies stored row patches.  It contains none of the method's arithmetic: no
head, tree, attention, verification or acceptance step is computed here.  Both
the CPU oracle and the GPU path consume the exact bytes it produces.
"""
from .configs import CONFIGS, Config, get_config
from .gen import (Inputs, bf16_bits_to_f32, f32_to_bf16_bits, integers, make_inputs,
                  normal_bf16)

__all__ = ["CONFIGS", "Config", "get_config", "Inputs", "make_inputs",
           "bf16_bits_to_f32", "f32_to_bf16_bits", "normal_bf16", "integers"]
