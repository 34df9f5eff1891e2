"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark."""
from .workloads import (SPECS, Spec, kv_head, kv_layer, needle_segment, planted_starts, queries,
                        retrieval_heads, seed_for, spec, spike_levels, surprisal, surprisal_batch,
                        torch_dtype, zoom_targets)

__all__ = ["SPECS", "Spec", "kv_head", "kv_layer", "needle_segment", "planted_starts", "queries",
           "retrieval_heads", "seed_for", "spec", "spike_levels", "surprisal", "surprisal_batch",
           "torch_dtype", "zoom_targets"]
