"""Seeded synthetic inputs for the quantized-expert MoE step.

This package is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It produces inputs only (codes, scales, biases, router weights,
activations, routing perturbations) and contains none of the method's
arithmetic. Every value is a pure function of integer keys, so the host
generator here and the device generator in ``gen_device.hip`` produce the same
bits.
"""
from .gen import *  # noqa: F401,F403
