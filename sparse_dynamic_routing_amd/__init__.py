"""Graph Machine sparse-layer hot path for AMD MI355X (gfx950).

Sparse edge referral (SER) and sparse edge attention (SEA), forward and
backward, as hand-written HIP kernels behind the C ABI of include/gm.h
(libgm.so).  This package is the thin Python binding of that library; see
``binding`` for the calls.  Importing the package does not load the library;
the first call does, and raises if it is not built.
"""
from .binding import (  # noqa: F401
    EXPORTS, GMError, check_edges, decode_step, gm_check_edges, gm_decode_step,
    gm_sea_backward, gm_sea_backward_noalloc, gm_sea_forward, gm_ser_sea_forward, ser_sea_forward,
    gm_sea_backward_workspace_bytes, gm_ser_backward, gm_ser_backward_workspace_bytes, gm_ser_forward,
    load, sea_backward, sea_forward, sea_workspace, ser_backward, ser_forward, ser_workspace,
    stats_as_query_heads, stats_edge_copy, stats_shape, gm_leg_mix_forward, gm_leg_mix_backward,
    gm_leg_mix_backward_workspace_bytes, leg_mix, leg_mix_backward, gm_dense_refresh,
    dense_refresh, gm_ser_forward_chain2, ser_forward_chain2,
)
