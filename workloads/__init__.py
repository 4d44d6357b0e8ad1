"""Seeded synthetic inputs for the POET-X linear layer.

This package only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no CNP, no block products, no merge).  Both the fp64 oracle
and the HIP path consume what it produces, bit for bit.
"""

from .configs import WORKLOADS, LinearShape, Workload, get_workload  # noqa: F401
from .gen import (  # noqa: F401
    LinearInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_linear_inputs,
    packed_len,
)
