"""Predictor-gated, neuron-aware sparse FFN for AMD Instinct MI355X (gfx950).

The compute path is libpi.so (HIP kernels behind the C ABI of include/pi.h);
`binding` is its ctypes wrapper and `layer` moves a layer's tensors to the
device and runs the decode step through it.
"""
from .binding import *  # noqa: F401,F403
