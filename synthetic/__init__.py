"""Seeded synthetic inputs for the routed MoE FFN layer.

This package holds only input recipes (shapes, seeds, value distributions).
It contains none of the layer's arithmetic, so both the CPU oracle's tests and
the GPU path's tests, bench and smoke run can draw identical inputs from it.
"""
from .moe_inputs import (  # noqa: F401
    CONFIGS,
    MoEConfig,
    MoEInputs,
    make_inputs,
    scaled_config,
)
from .latent_inputs import (  # noqa: F401
    LATENT_CONFIGS,
    LatentConfig,
    LatentInputs,
    make_latent_inputs,
    scaled_latent,
)
