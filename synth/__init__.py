"""Seeded synthetic inputs for the MoE layer, shared by the oracle tests, the HIP
parity tests, ``bench.py`` and the smoke check.

This module draws random numbers and nothing else: it holds none of the layer's
arithmetic (no routing, no planning, no expert math).  Every tensor comes from its
own torch generator seeded with ``seed * 1_000_003 + tensor_id`` so that each side
of a comparison can regenerate exactly the same values.
"""
from .inputs import CONFIGS, Shape, make_inputs, shape_of, zipf_bias  # noqa: F401
