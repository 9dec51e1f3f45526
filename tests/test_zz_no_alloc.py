"""The allocation-free SEA backward, gm_sea_backward_noalloc, through the C
ABI, against gm_sea_backward with a caller-provided workspace: the two run
the same kernels, so every output must be bitwise equal.  Two calls in a
row, the second on a smaller input (the fixed scratch keeps the first
call's contents, which must not matter), with the softmax recomputed and
with the forward's statistics."""
from __future__ import annotations

import pytest
import torch

import sparse_dynamic_routing_amd as gm
import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


def _inputs(B, n, hkv, G, d, s, seed, dtype=torch.bfloat16):
    idx, w = synth.edges(seed, B, n, hkv, s, mode="mixed")
    idx, w = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
    hq = G * hkv
    q = synth.normal(seed, "q", (B, n, hq, d), dtype, device="cuda")
    k = synth.normal(seed, "k", (B, n, hkv, d), dtype, device="cuda")
    v = synth.normal(seed, "v", (B, n, hkv, d), dtype, device="cuda")
    do = synth.normal(seed, "dout", (B, n, hq, d), dtype, device="cuda")
    ia, wa = gm.ser_forward(idx, w, idx, w, s)
    return q, k, v, ia, wa, do


def _grads(q, k, v, ia):
    f32 = dict(dtype=torch.float32, device="cuda")
    return (torch.full(q.shape, float("nan"), **f32), torch.full(k.shape, float("nan"), **f32),
            torch.full(v.shape, float("nan"), **f32), torch.full(ia.shape, float("nan"), **f32))


@pytest.mark.parametrize("with_stats", [False, True], ids=["recompute", "stats"])
def test_noalloc_backward_matches_workspace_call(with_stats):
    # the measured layer, then a smaller and ragged one
    for B, n, hkv, G, d, s in ((8, 4096, 8, 2, 128, 4), (2, 1500, 4, 3, 64, 4)):
        say(f"case noalloc stats={with_stats} B={B} n={n} hkv={hkv} G={G} d={d} s={s}")
        q, k, v, ia, wa, do = _inputs(B, n, hkv, G, d, s, synth.BASE_SEED + 50 + n)
        st = gm.sea_forward(q, k, v, ia, wa, save_stats=True)[1] if with_stats else None
        ref = _grads(q, k, v, ia)
        ws = gm.sea_workspace(q, ia)
        gm.gm_sea_backward(q, k, v, ia, wa, do, *ref, ws, stats=st)
        got = _grads(q, k, v, ia)
        gm.gm_sea_backward_noalloc(q, k, v, ia, wa, do, *got, stats=st)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dw"), got, ref):
            assert bool(torch.isfinite(b).all()), f"{name}: reference not fully written"
            assert torch.equal(a, b), f"{name}: allocation-free call differs"
        say("  dq, dk, dv, dw bitwise equal to the workspace call")
        del q, k, v, ia, wa, do, st, ref, got, ws
        torch.cuda.empty_cache()
