"""Seeded synthetic inputs for the MXFP8 publishing GEMM.

This package only draws random numbers and encodes them as MXFP8 bytes. It holds
none of the GEMM's, the rounding's or the mailbox's arithmetic, and it imports
neither the CPU oracle nor the HIP library: both sides consume the same bytes.
"""

from .generate import (  # noqa: F401
    CONFIGS,
    Problem,
    config_problem,
    config_seed,
    peer_payloads,
    quantize_mxfp8,
    random_problem,
)
