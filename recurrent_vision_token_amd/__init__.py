"""Chunkwise gated linear attention with key-only decay over a patch grid,
as hand-written HIP kernels for AMD Instinct MI355X (gfx950).

    out, final_state = gla_chunk_fwd(q, k, v, log_alpha, scan_dir)
    out, final_state = gla_chunk_fwd_ex(q, k, v, gate_logits, scan_dir,
                                        gate_mode="logits", tau=16.0,
                                        initial_state=state)
    gla_chunk_fwd_noalloc(q, k, v, log_alpha, scan_dir, out, final_state)
    dq, dk, dv, dla, _ = gla_chunk_bwd(q, k, v, log_alpha, d_out, scan_dir)
    h = spatial_swiglu(gate, value, weight, bias)   # the block's SwiGLU mixer
    o, kv = saga_fwd(q, k, v, alpha, beta)          # non-causal gated linear attention

The heavy lifting is in libgla.so (C ABI: include/gla.h); this package is a
thin binding around it plus the seeded synthetic workloads.
"""

from ._lib import (GlaError, gla_chunk_bwd, gla_chunk_fwd, gla_chunk_fwd_ex,  # noqa: F401
                   gla_chunk_fwd_noalloc, load, release_workspaces, saga_fwd, set_forward_mode, spatial_swiglu, status_str)

SCAN_L2R, SCAN_R2L, SCAN_T2B, SCAN_B2T, SCAN_ROTATE_BATCH = 0, 1, 2, 3, 4

__all__ = ["gla_chunk_fwd", "gla_chunk_fwd_ex", "gla_chunk_fwd_noalloc", "gla_chunk_bwd", "spatial_swiglu", "saga_fwd",
           "GlaError", "load", "release_workspaces", "set_forward_mode", "status_str", "SCAN_L2R",
           "SCAN_R2L", "SCAN_T2B", "SCAN_B2T", "SCAN_ROTATE_BATCH"]
