"""gm_ser_sea_forward (SER then SEA forward in one call, one fused kernel on
the measured shape) against the two calls it replaces and the oracle.

The fused kernel merges and ranks each unit's 16 two-hop candidates in a
16-lane row (fp64 sums in path order) and runs the SEA row kernel's
arithmetic on the kept slots, so A', o and the saved statistics must be
bitwise what gm_ser_forward followed by gm_sea_forward write."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cases
import oracle
import sparse_dynamic_routing_amd as gm
import synth
from gpu_util import TOL, Inputs, assert_close, assert_ser_match, dev, host, say

pytestmark = pytest.mark.gpu


def _two_calls(idx1, w1, idx2, w2, s1, q, k, v):
    io, wo = gm.ser_forward(idx1, w1, idx2, w2, s1)
    o, st = gm.sea_forward(q, k, v, io, wo, save_stats=True)
    return io, wo, o, st


def _check_equal(fused, ref):
    # bit patterns: the statistics of fp32 inputs hold fp64 values, whose
    # halves read as fp32 words can be NaN patterns
    for name, a, b in zip(("idx'", "w'", "o", "stats"), fused, ref):
        if a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        assert torch.equal(a, b), f"{name}: fused call differs from the two calls"


def test_fused_full_size_every_pair():
    """The measured layer (B = 8, n = 4096, 16 q / 8 KV heads, d = 128, bf16,
    s = 4/4/4): bitwise equal to the two calls; A' bit-exact and o within
    the bar against the oracle on every (batch, KV head) pair."""
    p = synth.PRESETS["ser_sea4"]
    say(f"case fused forward, full size {p}")
    inp = Inputs(p)
    idx, w = dev(inp.idx), dev(inp.w)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    fused = gm.ser_sea_forward(idx, w, idx, w, p.s1, q, k, v, save_stats=True)
    ref = _two_calls(idx, w, idx, w, p.s1, q, k, v)
    torch.cuda.synchronize()
    _check_equal(fused, ref)
    io, wo, o = host(fused[0]), host(fused[1]), host(fused[2])
    orc = oracle.get()
    G = p.hq // p.hkv
    worst = 0.0
    for b in range(p.B):
        for h in range(p.hkv):
            e_i, e_w = inp.idx[b:b + 1, :, h:h + 1], inp.w[b:b + 1, :, h:h + 1]
            ri, rw = orc.ser_forward(e_i, e_w, e_i, e_w, p.s1)
            assert (io[b:b + 1, :, h:h + 1] == ri).all(), f"A' indices differ in pair ({b}, {h})"
            assert (wo[b:b + 1, :, h:h + 1] == rw).all(), f"A' weights differ in pair ({b}, {h})"
            ro = orc.sea_forward(inp.host("q")[b:b + 1, :, h * G:(h + 1) * G],
                                 inp.host("k")[b:b + 1, :, h:h + 1],
                                 inp.host("v")[b:b + 1, :, h:h + 1], ri, rw)
            worst = max(worst, assert_close("o", o[b:b + 1, :, h * G:(h + 1) * G], ro,
                                            TOL[p.dtype], quiet=True)[0])
    say(f"  all pairs: A' bit-exact, o max scaled error {worst:.3e}")


SHAPES = [
    # B, n, hkv, G, d, s1, s2, s3, dtype, ties, pad (fused kernel or the two stages)
    (2, 67, 2, 2, 128, 4, 4, 4, torch.bfloat16, False, 0.1),    # ragged, padding slots
    (2, 70, 3, 1, 128, 4, 4, 4, torch.bfloat16, True, 0.0),     # exact ties: lower index first
    (1, 1, 2, 4, 128, 4, 4, 4, torch.bfloat16, False, 0.0),     # a single token
    (2, 45, 2, 8, 128, 4, 4, 4, torch.bfloat16, False, 0.2),
    (1, 33, 2, 16, 128, 4, 4, 4, torch.bfloat16, True, 0.1),
    (2, 50, 2, 2, 64, 4, 4, 4, torch.bfloat16, False, 0.1),     # other shapes: two stages
    (2, 50, 2, 2, 128, 2, 4, 4, torch.bfloat16, False, 0.1),
    (1, 40, 2, 3, 64, 3, 2, 3, torch.float32, True, 0.1),
]


@pytest.mark.parametrize("B,n,hkv,G,d,s1,s2,s3,dtype,ties,pad", SHAPES,
                         ids=[f"B{c[0]}-n{c[1]}-G{c[3]}-d{c[4]}-s{c[5]}{c[6]}{c[7]}-{str(c[8])[6:]}"
                              f"{'-ties' if c[9] else ''}" for c in SHAPES])
def test_fused_shapes(B, n, hkv, G, d, s1, s2, s3, dtype, ties, pad):
    say(f"case fused B={B} n={n} hkv={hkv} G={G} d={d} s={s1}/{s2}/{s3} {dtype} ties={ties}")
    rng = np.random.default_rng(n * 100 + G * 10 + s1)
    idx1, w1 = cases.edges(rng, B, n, hkv, s2, pad_frac=pad, ties=ties, dead_frac=0.05)
    idx2, w2 = cases.edges(rng, B, n, hkv, s3, pad_frac=pad, ties=ties, dead_frac=0.05)
    hq = G * hkv
    q = torch.from_numpy(rng.standard_normal((B, n, hq, d), dtype=np.float32)).to(dtype)
    k = torch.from_numpy(rng.standard_normal((B, n, hkv, d), dtype=np.float32)).to(dtype)
    v = torch.from_numpy(rng.standard_normal((B, n, hkv, d), dtype=np.float32)).to(dtype)
    args = [dev(x) for x in (idx1, w1, idx2, w2)]
    with_paths = max(s1, s2, s3) <= 4
    fused = gm.ser_sea_forward(*args, s1, dev(q), dev(k), dev(v), save_stats=True,
                               save_paths=with_paths)
    ref = _two_calls(*args, s1, dev(q), dev(k), dev(v))
    if with_paths:
        # the path map as gm_ser_forward writes it
        assert torch.equal(fused[4], gm.ser_forward(*args, s1, save_paths=True)[2])
        fused = fused[:4]
    again = gm.ser_sea_forward(*args, s1, dev(q), dev(k), dev(v), save_stats=True)
    torch.cuda.synchronize()
    _check_equal(fused, ref)
    _check_equal(again, fused)
    orc = oracle.get()
    ri, rw = orc.ser_forward(idx1, w1, idx2, w2, s1)
    assert_ser_match(host(fused[0]), host(fused[1]), ri, rw)
    np.testing.assert_array_equal(host(fused[1]), rw)
    assert_close("o", host(fused[2]), orc.sea_forward(q, k, v, ri, rw), TOL[dtype])
