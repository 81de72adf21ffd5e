"""sparse_long_context_piattn_amd -- pi-Attention forward on AMD MI355X.

The compute lives in libpiattn.so (HIP kernels for gfx950, C ABI in
include/piattn.h); this package is its thin Python binding plus the seeded
synthetic workloads used by the tests and the benchmark.
"""
from .binding import (Pattern, PiattnError, bwd, cache_append, decode, decode_workspace_bytes,
                      forced_kernels, fwd, fwd_noalloc, fwd_workspace_bytes, gate_logits, lib, make_pattern,
                      neighbors, neighbors_cap, out_proj, rolling_slots, version)

__all__ = ["Pattern", "PiattnError", "bwd", "cache_append", "decode", "decode_workspace_bytes",
           "forced_kernels", "fwd", "fwd_noalloc",
           "fwd_workspace_bytes", "gate_logits", "lib", "make_pattern", "neighbors", "neighbors_cap",
           "out_proj", "rolling_slots", "version"]
