"""Seeded synthetic inputs (counter-based RNG + the five workload recipes).

Shared by the CPU oracle and the GPU path; holds none of the layer's arithmetic."""
from . import rng
from .configs import CONFIGS, CONFIG_ORDER, DreamerConfig, make_bias, make_weights, make_x0

__all__ = ["rng", "CONFIGS", "CONFIG_ORDER", "DreamerConfig", "make_bias", "make_weights",
           "make_x0"]
