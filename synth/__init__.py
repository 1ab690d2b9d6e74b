"""Seeded synthetic workloads for the CCA / CCGQA forward pass.

This package is shared by the oracle tests, the GPU parity tests and the
benchmark.  It holds shapes, seeded random draws and the rounding of those
draws to the storage precision -- and nothing of the method's arithmetic
(no projection, convolution, normalisation, rotation or attention).
"""

from .configs import (CCAShape, COMPARISONS, COMPARISON_OVERRIDES, WORKLOADS,  # noqa: F401
                      shape_from_dict, workload)
from .generate import (  # noqa: F401
    Prefill,
    Decode,
    Backward,
    make_prefill,
    make_upstream_grad,
    add_chan_dense,
    make_decode,
    round_to_bf16_bits,
    bf16_bits_to_f64,
    f64_to_bf16_f64,
)
