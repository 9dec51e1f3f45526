"""GPU parity of leg construction (gm_leg_mix_forward / _backward) against
the oracle: legs bit-exact (indices and weights), dw and dalpha within 1e-5
(fp32 rounding of fp64 sums; dalpha sums up to B*n terms)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cases
import oracle
import sparse_dynamic_routing_amd as gm
from gpu_util import assert_close, assert_ser_match, dev, host, say

pytestmark = pytest.mark.gpu

LEG_CASES = [
    # B, n, hkv, K, s, ties
    (2, 70, 2, 16, 4, False),     # the stored-edge count of the K16 models
    (2, 70, 2, 16, 4, True),      # exact ties: lower index first
    (2, 70, 2, 16, 2, True),      # top-2 legs (the narrower budget), ties
    (1, 50, 3, 24, 4, False),     # K24: 32-lane teams
    (2, 33, 2, 5, 8, False),      # more slots than candidates: padding
    (1, 40, 1, 64, 16, True),     # a full wave per unit
    (3, 17, 2, 1, 2, False),      # one stored slot
    (8, 4096, 8, 16, 4, False),   # full size: B = 8, n = 4096, 8 KV heads
]


@pytest.mark.parametrize("B,n,hkv,K,s,ties", LEG_CASES,
                         ids=[f"B{c[0]}-n{c[1]}-h{c[2]}-K{c[3]}-s{c[4]}{'-ties' if c[5] else ''}"
                              for c in LEG_CASES])
def test_leg_mix_forward_backward(B, n, hkv, K, s, ties):
    say(f"case leg mix B={B} n={n} hkv={hkv} K={K} s={s} ties={ties}")
    rng = np.random.default_rng(B * 1000 + K * 10 + s)
    idx, w = cases.edges(rng, B, n, hkv, K, pad_frac=0.1, dead_frac=0.05, ties=ties)
    alpha = (rng.choice(cases.TIE_WEIGHTS, size=(hkv, K)) if ties
             else rng.random((hkv, K)) + 0.05).astype(np.float32)
    alpha[rng.random(alpha.shape) < 0.1] = 0.0
    io, wo = gm.leg_mix(dev(idx), dev(w), dev(alpha), s)
    dleg = rng.standard_normal((B, n, hkv, s)).astype(np.float32)
    dw, da = gm.leg_mix_backward(dev(idx), dev(w), dev(alpha), io, wo, dev(dleg))
    torch.cuda.synchronize()
    orc = oracle.get()
    rio, rwo = orc.leg_mix_forward(idx, w, alpha, s)
    assert_ser_match(host(io), host(wo), rio, rwo)
    np.testing.assert_array_equal(host(wo), rwo)
    rdw, rda = orc.leg_mix_backward(idx, w, alpha, rio, rwo, dleg)
    assert_close("dw", host(dw), rdw, 1e-5)
    assert_close("dalpha", host(da), rda, 1e-5)


def test_leg_mix_backward_deterministic():
    """dalpha is reduced in a fixed order: two runs agree bitwise."""
    rng = np.random.default_rng(3)
    idx, w = cases.edges(rng, 4, 1000, 4, 16)
    alpha = (rng.random((4, 16)) + 0.1).astype(np.float32)
    io, wo = gm.leg_mix(dev(idx), dev(w), dev(alpha), 4)
    dleg = dev(rng.standard_normal(io.shape).astype(np.float32))
    a = gm.leg_mix_backward(dev(idx), dev(w), dev(alpha), io, wo, dleg)
    b = gm.leg_mix_backward(dev(idx), dev(w), dev(alpha), io, wo, dleg)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_leg_mix_lane_and_team_kernels_agree():
    """K = 16 with 16-byte aligned rows takes the lane-per-unit kernel; the
    same rows one element off alignment take the 16-lane team kernel: both
    give the same bits (and the oracle's)."""
    rng = np.random.default_rng(21)
    B, n, hkv, K = 2, 300, 4, 16
    idx, w = cases.edges(rng, B, n, hkv, K, pad_frac=0.1, dead_frac=0.05, ties=True)
    alpha = rng.choice(cases.TIE_WEIGHTS, size=(hkv, K)).astype(np.float32)
    for s in (4, 2):
        io, wo = gm.leg_mix(dev(idx), dev(w), dev(alpha), s)
        # misaligned copies: rows start 4 bytes past a 16-byte boundary
        ib = torch.zeros(idx.size + 1, dtype=torch.int32, device="cuda")
        wb = torch.zeros(w.size + 1, dtype=torch.float32, device="cuda")
        im = ib[1:].view(idx.shape)
        wm = wb[1:].view(w.shape)
        im.copy_(dev(idx)); wm.copy_(dev(w))
        assert im.data_ptr() % 16 == 4
        io2, wo2 = gm.leg_mix(im, wm, dev(alpha), s)
        torch.cuda.synchronize()
        assert torch.equal(io, io2) and torch.equal(wo, wo2)
        rio, rwo = oracle.get().leg_mix_forward(idx, w, alpha, s)
        np.testing.assert_array_equal(host(io), rio)
        np.testing.assert_array_equal(host(wo), rwo)
        # backward: lane kernel (aligned) and team kernel (misaligned rows)
        dleg = rng.standard_normal(io.shape).astype(np.float32)
        dw, da = gm.leg_mix_backward(dev(idx), dev(w), dev(alpha), io, wo, dev(dleg))
        dw2, da2 = gm.leg_mix_backward(im, wm, dev(alpha), io, wo, dev(dleg))
        torch.cuda.synchronize()
        rdw, rda = oracle.get().leg_mix_backward(idx, w, alpha, rio, rwo, dleg)
        for name, got in (("dw lane", dw), ("dw team", dw2)):
            assert_close(name, host(got), rdw, 1e-5)
        for name, got in (("dalpha lane", da), ("dalpha team", da2)):
            assert_close(name, host(got), rda, 1e-5)
