"""fp64 CPU oracle for shifted local-window attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this package.
The HIP library neither imports nor links it, and it imports nothing from the library.
"""
from .basa_oracle import (  # noqa: F401
    check_partition,
    full_attention,
    full_attention_rows,
    members_of,
    reduce_shift,
    window_attention,
    window_attention_loops,
    window_attention_rows,
    window_members,
    window_weights,
)
