"""MI355X (gfx950) DSA lightning indexer -> top-k -> sparse MLA with cross-layer IndexShare.

The compute lives in libdsa.so (C ABI: include/dsa.h); ``binding`` marshals torch
tensors into it.  ``synth`` holds the seeded synthetic workloads.
"""
from . import binding  # noqa: F401
from .binding import (DsaError, IndexCache, group_forward, group_stats_compute, indexer_scores,  # noqa: F401
                      make_shape, sparse_mla_attention, topk_select, workspace_bytes)
