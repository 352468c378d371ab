"""Seeded synthetic inputs for the compressed-attention path.

This package only draws random numbers and stores them in the storage formats the
path consumes (fp32, bfloat16, OCP FP8 E4M3FN).  It holds none of the method's
arithmetic: no pooling, scoring, selection or attention.  Both the CPU oracle and the
GPU path are fed from here, so that they see identical input bytes.
"""
from .codecs import f32_to_bf16_bits, f32_to_e4m3fn_bits  # noqa: F401
from .configs import CONFIGS, Config, get_config  # noqa: F401
