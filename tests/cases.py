"""Small random edge cases for the pins: ties, padding slots, duplicates.

Only draws inputs (no SER/SEA arithmetic).  Weights drawn from a small set of
dyadic values make exact ties common, so the tie rule is exercised.
"""
from __future__ import annotations

import numpy as np

TIE_WEIGHTS = np.array([0.125, 0.25, 0.5, 1.0])


def edges(rng, B, n, hkv, s, pad_frac=0.0, ties=False, self_loop_frac=0.0, dead_frac=0.0):
    """Causal random edges.  ``pad_frac`` slots become padding (0, 0.0);
    ``dead_frac`` slots keep their index but get weight 0 (not an edge)."""
    i = np.arange(n).reshape(1, n, 1, 1)
    idx = np.floor(rng.random((B, n, hkv, s)) * (i + 1)).astype(np.int64)
    idx = np.minimum(idx, i)
    if self_loop_frac:
        idx = np.where(rng.random(idx.shape) < self_loop_frac, np.broadcast_to(i, idx.shape), idx)
    if ties:
        w = rng.choice(TIE_WEIGHTS, size=idx.shape)
    else:
        w = rng.random(idx.shape) + 1e-3
    if pad_frac:
        pad = rng.random(idx.shape) < pad_frac
        idx = np.where(pad, 0, idx)
        w = np.where(pad, 0.0, w)
    if dead_frac:
        w = np.where(rng.random(idx.shape) < dead_frac, 0.0, w)
    return idx.astype(np.int32), w.astype(np.float32)


def normal(rng, shape):
    return rng.standard_normal(shape)
