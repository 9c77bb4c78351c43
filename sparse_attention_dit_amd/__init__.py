"""MI355X-native shifted local-window attention (BASA, arXiv 2610.08772, §3.1).

The compute lives in the HIP library ``libbasa.so`` (C ABI: include/basa.h); this package
only marshals torch device tensors into it. Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from ._lib import (  # noqa: F401
    BasaError,
    full_attn_fwd,
    load,
    pool_kv,
    pooled_count,
    route_top1,
    shift_schedule,
    status_string,
    version,
    window_attn_fwd,
    window_attn_mem_fwd,
    window_attn_routed_fwd,
    window_means,
    window_perm,
)
