"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package only draws random numbers and stores them; it holds none of the
method's arithmetic. Floating-point draws are fp32; bf16 tensors are produced
from them by round-to-nearest-even on the bit pattern and kept as uint16
storage. `to_f64` widens stored values exactly (every bf16 and fp32 value is
representable in fp64), so the oracle sees exactly the values the GPU reads.
"""
from .inputs import *  # noqa: F401,F403
