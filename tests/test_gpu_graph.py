"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the four calls of a layer pass, then leg construction, the decode
step and the refresh edges.

Every call only launches kernels on the caller's stream (zero-fills are
kernels, not memsets; workspaces come from the caller), so a whole layer pass
can be captured once and replayed.  Each replay is checked against the eager
result of the same pass, with other eager work and synchronisations between
replays.  The SER gradients, fp64 sums whose order follows LDS atomics and
is rounded once to fp32 (two eager runs can differ in the last bit), are
compared to 1e-5 relative and absolute; everything else, dk and dv included
(each row summed over its incoming edges in edge-id order), must be
identical.
"""
from __future__ import annotations

import pytest
import torch

import sparse_dynamic_routing_amd as gm
import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


class LayerPass:
    """Inputs, preallocated outputs and workspaces of one SER+SEA fwd+bwd pass."""

    def __init__(self, B, n, hq=16, hkv=8, d=128, s=4, seed=synth.BASE_SEED + 40):
        idx, w = synth.edges(seed, B, n, hkv, s, mode="mixed")
        cu = lambda x: torch.from_numpy(x).cuda()  # noqa: E731
        self.idx, self.w = cu(idx), cu(w)
        qs, ks = (B, n, hq, d), (B, n, hkv, d)
        act = lambda name, shape: synth.normal(seed, name, shape, torch.bfloat16,  # noqa: E731
                                               device="cuda")
        self.q, self.k, self.v, self.dout = act("q", qs), act("k", ks), act("v", ks), act("dout", qs)
        f32 = dict(dtype=torch.float32, device="cuda")
        self.ia = torch.empty(idx.shape, dtype=torch.int32, device="cuda")
        self.wa = torch.empty(idx.shape, **f32)
        self.o = torch.empty_like(self.q)
        self.stats = torch.empty(gm.stats_shape(self.q, hkv, s), dtype=torch.float32,
                                 device="cuda")
        self.dq = torch.empty(qs, **f32)
        self.dk = torch.empty(ks, **f32)
        self.dv = torch.empty(ks, **f32)
        self.dwa = torch.empty(idx.shape, **f32)
        self.dA = torch.empty(idx.shape, **f32)
        self.paths = torch.empty(idx.shape[:3], dtype=torch.int64, device="cuda")
        self.ws_sea = gm.sea_workspace(self.q, self.ia)
        self.ws_ser = gm.ser_workspace(self.idx, self.idx, aliased=True)

    def outputs(self):
        return {"ia": self.ia, "wa": self.wa, "paths": self.paths, "o": self.o,
                "stats": self.stats, "dq": self.dq,
                "dk": self.dk, "dv": self.dv, "dwa": self.dwa, "dA": self.dA}

    def run(self):
        gm.gm_ser_forward(self.idx, self.w, self.idx, self.w, self.ia, self.wa, paths=self.paths)
        gm.gm_sea_forward(self.q, self.k, self.v, self.ia, self.wa, self.o, stats=self.stats)
        gm.gm_sea_backward(self.q, self.k, self.v, self.ia, self.wa, self.dout, self.dq, self.dk,
                           self.dv, self.dwa, self.ws_sea, stats=self.stats)
        gm.gm_ser_backward(self.idx, self.w, self.idx, self.w, self.ia, self.wa, self.dwa,
                           self.dA, self.dA, self.ws_ser, paths=self.paths)

    def poison(self):
        for t in self.outputs().values():
            if t.dtype in (torch.int32, torch.int64):
                t.fill_(-7)
            else:
                t.fill_(float("nan"))


ORDER_VARIES = {"dA"}


@pytest.mark.parametrize("B,n", [(2, 2048), (1, 8192)],
                         ids=["n2048-one-pass-index", "n8192-partitioned-index"])
def test_layer_pass_graph_replays_match_eager(B, n):
    say(f"case graph replay B={B} n={n}")
    lp = LayerPass(B, n)
    lp.run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in lp.outputs().items()}
    other = LayerPass(1, 512, seed=synth.BASE_SEED + 41)   # unrelated eager work

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lp.run()                                # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        lp.run()
    torch.cuda.synchronize()

    for rep in range(3):
        lp.poison()
        other.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        for name, t in lp.outputs().items():
            if name in ORDER_VARIES:
                err = (t - ref[name]).abs()
                bound = 1e-5 + 1e-5 * ref[name].abs()
                assert bool((err <= bound).all()), (
                    f"replay {rep}: {name} max |diff| {err.max().item():.3e}")
            else:
                assert torch.equal(t, ref[name]), f"replay {rep}: {name} differs from eager"


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_other_calls_graph_replays_match_eager():
    """Leg construction (forward and backward), the decode step, the refresh
    edges and two chained referral steps in one call captured together and
    replayed three times against the eager results (all bitwise: their sums
    run in a fixed order)."""
    say("case graph replay: leg construction, decode step, refresh edges, chained referral")
    B, n, hkv, hq, d, K, s = 2, 1024, 4, 8, 128, 16, 4
    seed = synth.BASE_SEED + 42
    cu = lambda x: torch.from_numpy(x).cuda()  # noqa: E731
    sidx, sw = synth.edges(seed, B, n, hkv, K, mode="mixed")
    sidx, sw = cu(sidx), cu(sw)
    alpha = torch.rand((hkv, K), generator=torch.Generator().manual_seed(5)).add_(0.05).cuda()
    eidx, ew = synth.edges(seed + 1, B, n, hkv, s, mode="mixed")
    eidx, ew = cu(eidx), cu(ew)
    q = synth.normal(seed, "q", (B, n, hq, d), torch.bfloat16, device="cuda")
    k = synth.normal(seed, "k", (B, n, hkv, d), torch.bfloat16, device="cuda")
    v = synth.normal(seed, "v", (B, n, hkv, d), torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {
        "li": torch.empty((B, n, hkv, s), dtype=torch.int32, device="cuda"),
        "lw": torch.empty((B, n, hkv, s), **f32),
        "dw": torch.empty((B, n, hkv, K), **f32),
        "da": torch.empty((hkv, K), **f32),
        "di": torch.empty((B, hkv, s), dtype=torch.int32, device="cuda"),
        "dwt": torch.empty((B, hkv, s), **f32),
        "do": torch.empty((B, hq, d), dtype=torch.bfloat16, device="cuda"),
        "ri": torch.empty((B, n, hkv, s), dtype=torch.int32, device="cuda"),
        "rw": torch.empty((B, n, hkv, s), **f32),
        "lse": torch.empty((B, n, hq), **f32),
        "c1i": torch.empty((B, n, hkv, s), dtype=torch.int32, device="cuda"),
        "c1w": torch.empty((B, n, hkv, s), **f32),
        "c2i": torch.empty((B, n, hkv, s), dtype=torch.int32, device="cuda"),
        "c2w": torch.empty((B, n, hkv, s), **f32),
    }
    dleg = synth.normal(seed + 7, "dout", (B, n, hkv, s), torch.float32, device="cuda")
    ws = torch.empty(max(gm.gm_leg_mix_backward_workspace_bytes(B, n, hkv, K), 8) // 8,
                     dtype=torch.float64, device="cuda")
    q1 = q[:, -1].contiguous()
    i1, w1 = eidx[:, -1].contiguous(), ew[:, -1].contiguous()

    def run():
        gm.gm_leg_mix_forward(sidx, sw, alpha, out["li"], out["lw"])
        gm.gm_leg_mix_backward(sidx, sw, alpha, out["li"], out["lw"], dleg, out["dw"],
                               out["da"], ws)
        gm.gm_decode_step(i1, w1, eidx, ew, q1, k, v, out["di"], out["dwt"], out["do"])
        gm.gm_dense_refresh(q, k, out["lse"], out["ri"], out["rw"])
        gm.gm_ser_forward_chain2(eidx, ew, out["c2i"], out["c2w"], out["c1i"], out["c1w"])

    run()
    torch.cuda.synchronize()
    ref = {name: t.clone() for name, t in out.items()}
    g = _capture(run)
    other = LayerPass(1, 512, seed=synth.BASE_SEED + 41)
    for rep in range(3):
        for t in out.values():
            if t.dtype == torch.int32:
                t.fill_(-7)
            else:
                t.fill_(float("nan"))
        other.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        for name, t in out.items():
            assert torch.equal(t, ref[name]), f"replay {rep}: {name} differs from eager"
