"""Seeded synthetic workloads for the MAC-Attention decode step.

This package holds only the workload shapes and the seeded random draws
(query streams, keys, values, outlier flags, contexts, page tables).  It
contains none of the method's arithmetic (no rotary embedding, no distance,
no softmax, no merge), so that both the fp64 oracle (``oracle/``) and the HIP
path (``kv_cache_reuse_amd``) can consume the very same inputs while sharing
no code with each other.
"""

from .streams import (  # noqa: F401
    WORKLOADS,
    Workload,
    Inputs,
    make_inputs,
    make_q_stream,
    workload,
)
