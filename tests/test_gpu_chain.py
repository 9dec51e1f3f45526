"""gm_ser_forward_chain2 (two chained referral steps in one launch) against
two gm_ser_forward calls and against the oracle.

A2 = Sp(A1 A1) with A1 = Sp(A0 A0) (ai.info "Graph Machine: Towards Better
Pretraining via Edges", Key Contributions 2: the edge matrix raised to a
power, one referral step per factor).  The fused kernel recomputes the rows
of A1 it needs with the arithmetic of one referral step, so A1 and A2 must
be bitwise what the two separate calls write, and the oracle's two steps
must match them (indices exact, weights bitwise)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cases
import oracle
import sparse_dynamic_routing_amd as gm
import synth
from gpu_util import assert_ser_match, dev, host, say

pytestmark = pytest.mark.gpu


def _bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    return torch.equal(a, b)


def _check(idx: np.ndarray, w: np.ndarray, oracle_check: bool = True):
    s = idx.shape[-1]
    di, dw = dev(idx), dev(w)
    i2, w2, i1, w1 = gm.ser_forward_chain2(di, dw, save_mid=True)
    j2, v2 = gm.ser_forward_chain2(di, dw)
    r1i, r1w = gm.ser_forward(di, dw, di, dw, s)
    r2i, r2w = gm.ser_forward(r1i, r1w, r1i, r1w, s)
    torch.cuda.synchronize()
    for name, a, b in (("A1 idx", i1, r1i), ("A1 w", w1, r1w), ("A2 idx", i2, r2i),
                       ("A2 w", w2, r2w), ("A2 idx (no A1)", j2, r2i),
                       ("A2 w (no A1)", v2, r2w)):
        assert _bits_equal(a, b), f"{name}: fused chain differs from two gm_ser_forward calls"
    if not oracle_check:
        return
    orc = oracle.get()
    o1i, o1w = orc.ser_forward(idx, w, idx, w, s)
    o2i, o2w = orc.ser_forward(o1i, o1w, o1i, o1w, s)
    assert_ser_match(host(i1), host(w1), o1i, o1w)
    assert_ser_match(host(i2), host(w2), o2i, o2w)
    np.testing.assert_array_equal(host(w2), o2w)


SHAPES = [
    # B, n, hkv, s, ties, pad, dead, self-loops
    (1, 1, 2, 4, False, 0.0, 0.0, 0.0),      # one token: every edge is (0, w)
    (2, 67, 3, 4, False, 0.1, 0.05, 0.0),    # ragged, padding and dead slots
    (2, 70, 2, 4, True, 0.0, 0.0, 0.0),      # exact ties: lower index first
    (3, 129, 2, 4, False, 0.0, 0.0, 0.5),    # many self loops: duplicate targets
    (1, 64, 2, 2, False, 0.0, 0.0, 0.0),     # the tiny configuration's width
    (2, 45, 3, 2, True, 0.2, 0.05, 0.1),
]


@pytest.mark.parametrize("B,n,hkv,s,ties,pad,dead,selfl", SHAPES,
                         ids=[f"B{c[0]}-n{c[1]}-h{c[2]}-s{c[3]}{'-ties' if c[4] else ''}"
                              f"{'-self' if c[7] else ''}" for c in SHAPES])
def test_chain2_shapes(B, n, hkv, s, ties, pad, dead, selfl):
    say(f"case chain2 B={B} n={n} hkv={hkv} s={s} ties={ties} pad={pad} dead={dead} "
        f"self={selfl}")
    rng = np.random.default_rng(n * 10 + s)
    idx, w = cases.edges(rng, B, n, hkv, s, pad_frac=pad, ties=ties, self_loop_frac=selfl,
                         dead_frac=dead)
    _check(idx, w)


def test_chain2_stack21_layer():
    """The 21-layer stack's edges (B = 32, n = 4096, 8 KV heads, s = 4, half
    local / half far): two steps fused, against the two calls and the
    oracle on every unit."""
    p = synth.PRESETS["stack21"]
    say(f"case chain2 full size {p.name}: B={p.B} n={p.n} hkv={p.hkv} s={p.s1}")
    idx, w = synth.edges(p.seed, p.B, p.n, p.hkv, p.s_in, mode=p.mode)
    _check(np.asarray(idx), np.asarray(w))


def test_chain2_long_context():
    """n = 65,536 (far edges over the whole prefix): against the two calls."""
    p = synth.PRESETS["long64k"]
    say(f"case chain2 long context B={p.B} n={p.n} hkv={p.hkv}")
    idx, w = synth.edges(p.seed, p.B, p.n, p.hkv, p.s_in, mode=p.mode)
    _check(np.asarray(idx), np.asarray(w), oracle_check=False)
