"""CPU oracle for the routed sparse causal attention path (TEST INFRASTRUCTURE).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package.  The product library never imports, links or runs it, and it
imports nothing from the product package.

`oracle.c` holds the algorithm (plain C, fp32 routing decisions, fp64
attention); `dense_twin.py` holds an independently written dense-mask twin of
the attention step in numpy.  Page citations are at each function in those
files.  Every function is pinned by tests under tests/ (brute force, closed
forms, library routines, invariants).
"""
from .binding import (  # noqa: F401
    Shape,
    build_oracle,
    load,
    rope_table,
    block_addresses,
    posting_lists,
    build_index,
    route,
    attention,
    num_addresses,
    max_threads,
    mixer,
    calibrate,
)
from .dense_twin import dense_masked_attention, dense_causal_attention  # noqa: F401
