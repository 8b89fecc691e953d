"""Workload definitions and seeded synthetic inputs.

This package holds only shapes, flags and random-number draws. It contains no
arithmetic of the transformer forward, so both the CPU oracle and the GPU path
can take their inputs from it without sharing any of the computation.
"""
from .configs import ModelConfig, CONFIGS, config_by_name  # noqa: F401
from .synth import synth_weights, synth_ids, weight_slots  # noqa: F401
