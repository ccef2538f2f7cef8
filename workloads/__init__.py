"""Seeded synthetic inputs for the block-FP8 mixture-of-experts expert computation.

This package only draws random inputs and lays them out in memory. It holds none of the
computation being tested: no e4m3 decoding, no routing, no GEMM, no activation. The
float64 oracle and the HIP library both consume what it produces, and neither is
imported here.
"""

from .gen import (  # noqa: F401
    DEFAULT_T,
    SHAPES,
    FP8Bank,
    MoECase,
    finite_e4m3_codes,
    bank_bytes_touched,
    make_bank,
    make_banks,
    make_case,
    make_hidden,
    make_logits,
    scale_cols_padded,
)
