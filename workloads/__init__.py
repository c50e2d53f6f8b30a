"""Seeded synthetic inputs for the TTQ linear projection.

This package only draws random numbers and rounds them to bfloat16 bit
patterns.  It holds none of the method's arithmetic, so both the CPU oracle
and the HIP path can consume the same bytes without sharing any code of the
method itself.
"""
from .configs import (  # noqa: F401
    Problem,
    bf16_round_bits,
    make_problem,
    make_c1,
    make_c2,
    make_c3,
    make_c4,
    make_c5,
    C5_PROJECTIONS,
)
