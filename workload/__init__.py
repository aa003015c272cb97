"""Seeded synthetic workloads shared by the oracle and the GPU path (inputs only)."""
from .synth import *  # noqa: F401,F403
from .synth import WORKLOADS, Workload, Layer, make_layer, make_x, make_profile_x  # noqa: F401
