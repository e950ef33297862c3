"""Seeded synthetic workloads shared by the tests, the bench and the CPU oracle.

This package holds shapes, mask parameters and a seeded input generator only.
It contains none of the method's arithmetic (no rotary encoding, no masking,
no attention): both the HIP path and the CPU oracle consume what it produces,
and neither imports the other.
"""
from .configs import WORKLOADS, Workload, MaskSpec, get_workload  # noqa: F401
from .synth import make_inputs, bf16_round, bf16_bits  # noqa: F401
