"""Seeded synthetic inputs shared by the tests, the bench and the smoke run.

This module holds no arithmetic of the attention method: it only draws
random tensors and casts them to bf16 (with torch's round-to-nearest-even
cast), so that the HIP path and the CPU oracle receive identical inputs.
"""
from .synthetic import CONFIGS, make_inputs, make_config_inputs  # noqa: F401
