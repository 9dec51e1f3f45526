"""GPU parity: the HIP path (through the C ABI) against the oracle.

Every stage is local to a (batch, KV head) pair, so the oracle recomputes
each pair of a full-size run exactly; the full-size presets are compared on
every pair, element by element (the 21-layer stack on sampled pairs through
all its layers).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_dynamic_routing_amd as gm
import synth
from gpu_util import (TOL, Inputs, assert_close, assert_ser_match, compare_pair, dev, download,
                      host, pairs_for, run_gpu, run_oracle_pair, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("stats", [False, True], ids=["recompute", "stats"])
def test_tiny_preset_whole_chain(stats):
    """tiny: batch 1, n=64, 4 q / 2 KV heads, d=16, fp32, s=2; one SER step
    then SEA forward and backward, then SER backward; all outputs compared."""
    p = synth.PRESETS["tiny"]
    say(f"case tiny stats={stats} {p}")
    inp = Inputs(p)
    got = run_gpu(inp, stats=stats)
    for b, h in pairs_for(p.B, p.hkv, count=p.B * p.hkv):
        say(f"  pair b={b} h={h}")
        compare_pair(p, got, run_oracle_pair(inp, b, h), b, h)


FULL = [("sea2", False), ("ser_sea4", True), ("metric", False), ("metric", True),
        ("long64k", True), ("theia", True), ("d64", True), ("d256", True), ("fp32", True)]


@pytest.mark.parametrize("name,stats", FULL,
                         ids=[f"{n}{'-stats' if s else ''}" for n, s in FULL])
def test_full_size_preset_every_pair(name, stats):
    """Every (batch, KV head) pair of the full-size run against the oracle,
    element by element.  stats: the forward saves p / w and the backward
    uses it (as the measured pass does).  The worst scaled and absolute
    error of each output over all pairs is printed."""
    p = synth.PRESETS[name]
    say(f"case {name} stats={stats} {p}")
    inp = Inputs(p)
    got = download(run_gpu(inp, stats=stats))
    torch.cuda.empty_cache()
    worst = {}
    for b in range(p.B):
        for h in range(p.hkv):
            compare_pair(p, got, run_oracle_pair(inp, b, h), b, h, worst=worst, quiet=True)
    say(f"  all {p.B * p.hkv} pairs within the bar (X = {TOL[p.dtype]:g}); worst over them:")
    for out, e in worst.items():
        if isinstance(e, tuple):
            say(f"    {out}: max scaled error {e[0]:.3e}, max absolute error {e[1]:.3e}")
        else:
            say(f"    {out}: {e}")


@pytest.mark.parametrize("name", ["ser_sea4", "theia"])
def test_ser_forward_full_size_every_row(name):
    """SER forward of the 4096-token presets (top-4 and top-2 of 16): every
    row bit-exact."""
    p = synth.PRESETS[name]
    idx, w = synth.edges(p.seed, p.B, p.n, p.hkv, p.s2, mode=p.mode)
    say(f"case ser_forward full {idx.shape}")
    io, wo = gm.ser_forward(dev(idx), dev(w), dev(idx), dev(w), p.s1)
    rio, rwo = oracle.get().ser_forward(idx, w, idx, w, p.s1)
    assert_ser_match(host(io), host(wo), rio, rwo)
    np.testing.assert_array_equal(host(wo), rwo)


def test_stack21_chained_layers_sampled_pairs():
    """21 sparse layers, each two chained SER steps (A <- Sparsify(A A)) then
    SEA, edges carried between layers, fresh q/k/v per layer (drawn on the
    GPU; the oracle gets the downloaded pair).  Edges must stay bit-exact
    through all 42 SER steps."""
    p = synth.PRESETS["stack21"]
    say(f"case stack21 {p}")
    G = p.hq // p.hkv
    idx0, w0 = synth.edges(p.seed, p.B, p.n, p.hkv, p.s2, mode=p.mode)
    pairs = pairs_for(p.B, p.hkv, count=2)
    orc = oracle.get()
    ia, wa = dev(idx0), dev(w0)
    ref_edges = {bh: (idx0[bh[0]:bh[0] + 1, :, bh[1]:bh[1] + 1].copy(),
                      w0[bh[0]:bh[0] + 1, :, bh[1]:bh[1] + 1].copy()) for bh in pairs}
    X = TOL[p.dtype]
    for layer in range(p.layers):
        for _ in range(p.ser_steps):
            ia, wa = gm.ser_forward(ia, wa, ia, wa, p.s1)
        q = synth.normal(p.seed, "q", (p.B, p.n, p.hq, p.d), p.dtype, layer, "cuda")
        k = synth.normal(p.seed, "k", (p.B, p.n, p.hkv, p.d), p.dtype, layer, "cuda")
        v = synth.normal(p.seed, "v", (p.B, p.n, p.hkv, p.d), p.dtype, layer, "cuda")
        o = gm.sea_forward(q, k, v, ia, wa)
        torch.cuda.synchronize()
        check = layer in (0, 1, p.layers // 2, p.layers - 1)
        if check:
            say(f"  layer {layer}")
        for (b, h) in pairs:
            ri, rw = ref_edges[(b, h)]
            for _ in range(p.ser_steps):
                ri, rw = orc.ser_forward(ri, rw, ri, rw, p.s1)
            ref_edges[(b, h)] = (ri, rw)
            if not check:
                continue
            gi = host(ia[b:b + 1, :, h:h + 1]); gw = host(wa[b:b + 1, :, h:h + 1])
            assert_ser_match(gi, gw, ri, rw)
            ro = orc.sea_forward(host(q[b:b + 1, :, h * G:(h + 1) * G]),
                                 host(k[b:b + 1, :, h:h + 1]), host(v[b:b + 1, :, h:h + 1]),
                                 ri, rw)
            assert_close(f"o layer {layer} pair ({b},{h})",
                         host(o[b:b + 1, :, h * G:(h + 1) * G]), ro, X)
        del q, k, v, o
