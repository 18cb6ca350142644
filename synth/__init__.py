"""Seeded synthetic inputs for sparse-times-dense products.

This package only draws random numbers and converts them to 16-bit storage
formats.  It holds none of the SpMM arithmetic and none of the sparse-format
construction, so both the CPU oracle and the GPU path can consume its output
without sharing code with each other.
"""

from .generators import (  # noqa: F401
    Problem,
    bf16_bits,
    config1,
    config2,
    config3_matrix,
    config3_specs,
    config4,
    config5,
    fp16_bits,
    make_dense_b,
    random_problem,
    block_problem,
    rng_for,
)
