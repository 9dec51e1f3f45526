"""Helpers shared by the GPU parity tests: running the HIP path for a preset,
running the oracle on one (batch, KV head) pair, and the tolerances.

Every stage of the path is local to a (batch b, KV head h) pair: SER reads
only rows of the same pair, SEA gathers K/V rows of the same pair and
scatters dk/dv back into it.  So the oracle can recompute any pair of a
full-size run exactly, from the same generated inputs, on its own.

Tolerances (the parity bar): SER indices bit-exact (rows whose s1-th and
(s1+1)-th oracle weights are within 1e-6 relative may differ), SER weights
within 1e-5 relative; SEA outputs and gradients within X * max(1, |ref|)
with X = 2e-2 for bf16 inputs and 1e-5 for fp32 inputs (plain absolute for
|ref| <= 1, relative above, since dw = dl / w grows large for small w).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_dynamic_routing_amd as gm
import synth

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype=None):
    t = torch.as_tensor(x) if not isinstance(x, torch.Tensor) else x
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def scaled_errors(got, ref):
    """(max scaled error |got - ref| / max(1, |ref|), max absolute error)."""
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not got.size:
        return 0.0, 0.0
    diff = np.abs(got - ref)
    return float((diff / np.maximum(1.0, np.abs(ref))).max()), float(diff.max())


def assert_close(name, got, ref, X, quiet=False):
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    worst = float(err.max()) if err.size else 0.0
    worst_abs = float(np.abs(got - ref).max()) if err.size else 0.0
    if not quiet:
        say(f"    {name}: max scaled error {worst:.3e}, max absolute error {worst_abs:.3e} "
            f"(bar {X:g})")
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert worst <= X, f"{name}: max scaled error {worst:.3e} > {X:g} at " \
        f"{np.unravel_index(int(err.argmax()), err.shape)}"
    return worst, worst_abs


def assert_ser_match(io, wo, rio, rwo, rwe=None, rel=1e-6):
    """Rows bit-exact, except near ties of the reference's s1-th/(s1+1)-th key
    (only computable when the caller passes the reference's candidate keys;
    the GPU sums in the definition's order and precision, so none is
    expected)."""
    io = np.asarray(io); rio = np.asarray(rio)
    bad = ~(io == rio).all(-1)
    nbad = int(bad.sum())
    say(f"    SER rows differing in indices: {nbad} of {bad.size}")
    assert nbad == 0, f"first differing row {np.argwhere(bad)[0].tolist()}: " \
        f"{io[tuple(np.argwhere(bad)[0])]} vs {rio[tuple(np.argwhere(bad)[0])]}"
    np.testing.assert_allclose(np.asarray(wo), np.asarray(rwo), rtol=1e-5, atol=0)
    exact = int((np.asarray(wo) == np.asarray(rwo)).all(-1).sum())
    say(f"    SER rows with bit-identical weights: {exact} of {bad.size}")


def pairs_for(B, hkv, count=3, seed=0):
    rng = np.random.default_rng(seed)
    ps = [(0, 0), (B - 1, hkv - 1)]
    while len(ps) < count and len(set(ps)) < B * hkv:
        ps.append((int(rng.integers(B)), int(rng.integers(hkv))))
    return sorted(set(ps))


def pair(x: np.ndarray, b: int, h: int, G: int = 0):
    """Slice one (b, h) pair: edges/k/v by KV head, q-shaped tensors by the
    group's query heads when G > 0."""
    if G:
        return np.ascontiguousarray(x[b:b + 1, :, h * G:(h + 1) * G])
    return np.ascontiguousarray(x[b:b + 1, :, h:h + 1])


class Inputs:
    """The seeded inputs of a preset (host numpy for the oracle, device for
    the HIP path)."""

    def __init__(self, p: synth.Preset, layer: int = 0, device_gen: bool = False):
        self.p = p
        idx, w = synth.edges(p.seed, p.B, p.n, p.hkv, p.s_in, mode=p.mode, layer=layer)
        self.idx, self.w = idx, w
        qs, ks = (p.B, p.n, p.hq, p.d), (p.B, p.n, p.hkv, p.d)
        where = "cuda" if device_gen else "cpu"
        self.q = synth.normal(p.seed, "q", qs, p.dtype, layer, where)
        self.k = synth.normal(p.seed, "k", ks, p.dtype, layer, where)
        self.v = synth.normal(p.seed, "v", ks, p.dtype, layer, where)
        self.dout = synth.normal(p.seed, "dout", qs, p.dtype, layer, where) if p.backward else None
        self._host = {}

    def host(self, name: str) -> np.ndarray:
        """An activation as host fp32 numpy, converted once."""
        if name not in self._host:
            self._host[name] = host(getattr(self, name))
        return self._host[name]


def run_gpu(inp: Inputs, stats: bool = False):
    """One pass of the path on the GPU; returns device tensors by name.  With
    ``stats`` the forward saves its p / w statistics and the SER path map, and
    the backward uses them."""
    p = inp.p
    out = {}
    idx, w = dev(inp.idx), dev(inp.w)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    paths = None
    if p.ser:
        # with saved state (stats) the forward also writes the path map for
        # the SER backward, as the measured pass does
        if stats and max(p.s1, p.s2, p.s3) <= 4:
            ia, wa, paths = gm.ser_forward(idx, w, idx, w, p.s1, save_paths=True)
        else:
            ia, wa = gm.ser_forward(idx, w, idx, w, p.s1)
        out["idx"], out["w"] = ia, wa
    else:
        ia, wa = idx, w
    st = None
    if stats:
        out["o"], st = gm.sea_forward(q, k, v, ia, wa, save_stats=True)
        out["stats"] = st
    else:
        out["o"] = gm.sea_forward(q, k, v, ia, wa)
    if p.backward:
        do = dev(inp.dout)
        dq, dk, dv, dw = gm.sea_backward(q, k, v, ia, wa, do, stats=st)
        out.update(dq=dq, dk=dk, dv=dv, dwp=dw)
        if p.ser:
            dA, _ = gm.ser_backward(idx, w, idx, w, ia, wa, dw, aliased=True, paths=paths)
            out["dA"] = dA
    torch.cuda.synchronize()
    return out


def run_oracle_pair(inp: Inputs, b: int, h: int):
    """The same pass by the oracle, for one (b, h) pair."""
    p = inp.p
    orc = oracle.get()
    G = p.hq // p.hkv
    idx, w = pair(inp.idx, b, h), pair(inp.w, b, h)
    q = pair(inp.host("q"), b, h, G)
    k, v = pair(inp.host("k"), b, h), pair(inp.host("v"), b, h)
    ref = {}
    if p.ser:
        ia, wa = orc.ser_forward(idx, w, idx, w, p.s1)
        ref["idx"], ref["w"] = ia, wa
    else:
        ia, wa = idx, w
    ref["o"], ref["p"] = orc.sea_forward(q, k, v, ia, wa, probs=True)
    ref["live"] = np.repeat(wa > 0, G, axis=2)
    ref["wq"] = np.repeat(wa, G, axis=2)          # each query head's slot weights
    if p.backward:
        do = pair(inp.host("dout"), b, h, G)
        dq, dk, dv, dw = orc.sea_backward(q, k, v, ia, wa, do)
        ref.update(dq=dq, dk=dk, dv=dv, dwp=dw)
        if p.ser:
            dA, _ = orc.ser_backward(idx, w, idx, w, ia, wa, dw, aliased=True)
            ref["dA"] = dA
    return ref


def download(got: dict) -> dict:
    """Every output of run_gpu as host numpy (statistics per query head)."""
    out = {}
    for name, t in got.items():
        if name == "stats":
            t = gm.stats_as_query_heads(t, got["o"].shape[2] // t.shape[1])
        out[name] = host(t)
    return out


def compare_pair(p: synth.Preset, got: dict, ref: dict, b: int, h: int, worst=None,
                 quiet=False):
    """One (b, h) pair of a run against the oracle's recomputation of it.
    ``got`` holds device tensors or (faster for many pairs) their download().
    ``worst``, when given, collects the largest (scaled, absolute) error of
    each output over the pairs compared."""
    G = p.hq // p.hkv
    X = TOL[p.dtype]
    hst = lambda name: got[name] if isinstance(got[name], np.ndarray) else (  # noqa: E731
        host(gm.stats_as_query_heads(got[name], G)) if name == "stats" else host(got[name]))

    def check(name, g, r, bar):
        e = assert_close(name, g, r, bar, quiet=quiet)
        if worst is not None:
            w0 = worst.get(name, (0.0, 0.0))
            worst[name] = (max(w0[0], e[0]), max(w0[1], e[1]))

    if "idx" in ref:
        if quiet:
            gi, gw = pair(hst("idx"), b, h), pair(hst("w"), b, h)
            assert (gi == ref["idx"]).all(), f"SER indices differ in pair ({b}, {h})"
            np.testing.assert_allclose(gw, ref["w"], rtol=1e-5, atol=0)
            if worst is not None:
                worst["SER rows not bit-identical"] = worst.get(
                    "SER rows not bit-identical", 0) + int((gw != ref["w"]).any(-1).sum())
        else:
            assert_ser_match(pair(hst("idx"), b, h), pair(hst("w"), b, h), ref["idx"], ref["w"])
    check("o", pair(hst("o"), b, h, G), ref["o"], X)
    if "stats" in got:
        # p / w per slot: times the GPU's own slot weights it is p
        st = pair(hst("stats"), b, h, G)
        assert (st[~ref["live"]] == 0).all(), "statistics of dead slots must be 0"
        wq = np.repeat(pair(hst("w"), b, h), G, axis=2) if "w" in got else ref["wq"]
        check("p (statistics * w)", st * wq, ref["p"], 1e-4)
    if "dq" in ref:
        check("dq", pair(hst("dq"), b, h, G), ref["dq"], X)
        check("dk", pair(hst("dk"), b, h), ref["dk"], X)
        check("dv", pair(hst("dv"), b, h), ref["dv"], X)
        check("dw (SEA)", pair(hst("dwp"), b, h), ref["dwp"], X)
    if "dA" in ref:
        check("dw (SER)", pair(hst("dA"), b, h), ref["dA"], X)
