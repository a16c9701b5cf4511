"""fp64 CPU oracle of the ETA decode step.

TEST INFRASTRUCTURE ONLY. This package is the independent reference that the
HIP path is checked against. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does. It
shares no code with the HIP library and imports nothing from it.

See `eta_oracle` for the method and the passages each step follows.
"""
from .eta_oracle import (  # noqa: F401
    BLOCK,
    upcast,
    sigmoid,
    gate,
    block_summary,
    build_summaries,
    threshold,
    block_bound,
    admitted_blocks,
    filtered_attention,
    decode,
    DecodeResult,
)
