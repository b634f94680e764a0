"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package draws random numbers and nothing else: it holds none of the
ternary method's arithmetic (no scale, no rounding to trits, no packing, no
product).  Both the fp64 oracle and the HIP library are fed from here, and
neither of them is imported by it.
"""

from .generators import (  # noqa: F401
    seed_for,
    activations_fp16,
    latent_weights_f32,
    ternary_iid,
    block_scales_fp16,
    BLOCK,
)
