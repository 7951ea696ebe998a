"""Seeded synthetic workloads for the paged KV attention tests and benchmark.

This module only draws inputs: lengths, page placement, the metadata an
engine's host side hands to the attention backend (block tables, slot
mappings, positions, cu_seqlens, context lengths) and the raw element bits of
q, k, v and the norm weights.  It holds none of the attention, norm or RoPE
arithmetic and imports neither the oracle nor the HIP library; both sides
consume what it returns.
"""

from .configs import (  # noqa: F401
    Workload, RequestData, make_workload, make_custom, config_names, CONFIGS,
    bf16_from_f32, sentinel_pool,
)
