"""Pins of the oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself:
  * dense n x n references (tests/dense_ref.py): SER as the product of two soft
    adjacency matrices then top-s1, SEA as masked causal attention with bias
    ln w (page "Graph Machine: Towards Better Pretraining via Edges", ai.info,
    Key Contributions 2-3, Methodology);
  * central finite differences of the oracle's own forward (gradients);
  * closed forms of special cases and exact invariants;
  * the KV-access fractions printed on the same page (Main Findings, "KV
    access reduction"), stored in tests/golden/kv_access.json.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import cases
import dense_ref
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _near_tie(kth, nxt, rel=1e-6):
    return (kth > 0) & (nxt > 0) & (np.abs(kth - nxt) <= rel * np.maximum(kth, nxt))


def assert_ser_equal(io, wo, ref_io, ref_wo, kth=None, nxt=None, wrel=1e-6):
    """Indices bit-exact and weights within ``wrel``, except rows whose s1-th
    and (s1+1)-th reference keys are within 1e-6 relative (near ties)."""
    exempt = np.zeros(io.shape[:3], bool) if kth is None else _near_tie(kth, nxt)
    ok_idx = (io == ref_io).all(-1) | exempt
    bad = np.argwhere(~ok_idx)
    assert bad.size == 0, f"{len(bad)} rows differ in indices, first {bad[:3].tolist()}: " \
        f"{io[tuple(bad[0])]} vs {ref_io[tuple(bad[0])]}"
    rows = ~exempt
    np.testing.assert_allclose(wo[rows], ref_wo[rows], rtol=wrel, atol=0)


# ---------------------------------------------------------------- SER forward
@pytest.mark.parametrize("mode", ["uniform", "mixed"])
def test_ser_forward_matches_dense_product(orc, mode):
    idx, w = synth.edges(7, B=2, n=96, hkv=2, s=4, mode=mode)
    io, wo = orc.ser_forward(idx, w, idx, w, s1=4)
    ref_io, ref_wo, kth, nxt = dense_ref.ser_forward(idx, w, idx, w, 4)
    assert_ser_equal(io, wo, ref_io, ref_wo, kth, nxt)


def test_ser_forward_tiny_config_dense(orc):
    p = synth.PRESETS["tiny"]
    idx, w = synth.edges(p.seed, p.B, p.n, p.hkv, p.s2, mode=p.mode)
    io, wo = orc.ser_forward(idx, w, idx, w, s1=p.s1)
    ref_io, ref_wo, kth, nxt = dense_ref.ser_forward(idx, w, idx, w, p.s1)
    assert_ser_equal(io, wo, ref_io, ref_wo, kth, nxt)


def test_ser_forward_1000_random_small_cases(orc):
    """Random shapes, two distinct legs, padding slots, zero-weight slots at
    non-zero indices, duplicates and exact ties (dyadic weights): the tie rule
    (lower index first) and "zero entries are not edges" must agree."""
    rng = np.random.default_rng(1000)
    for case in range(1000):
        B, hkv = rng.integers(1, 3, size=2)
        n = int(rng.integers(1, 24))
        s1, s2, s3 = (int(x) for x in rng.integers(1, 6, size=3))
        ties = bool(case % 2)
        dead = 0.2 * (case % 7 == 0)
        idx1, w1 = cases.edges(rng, B, n, hkv, s2, pad_frac=0.2 * (case % 3 == 0), ties=ties,
                               dead_frac=dead)
        idx2, w2 = cases.edges(rng, B, n, hkv, s3, pad_frac=0.2 * (case % 5 == 0), ties=ties,
                               dead_frac=dead)
        io, wo = orc.ser_forward(idx1, w1, idx2, w2, s1=s1)
        ref_io, ref_wo, kth, nxt = dense_ref.ser_forward(idx1, w1, idx2, w2, s1)
        if ties:   # dyadic sums are exact: no exemption at all
            np.testing.assert_array_equal(io, ref_io, err_msg=f"case {case}")
            np.testing.assert_array_equal(wo, ref_wo, err_msg=f"case {case}")
        else:
            assert_ser_equal(io, wo, ref_io, ref_wo, kth, nxt)


def test_ser_forward_pointer_chase_closed_form(orc):
    """s2 = s3 = 1: A' row i is the single path i -> j -> idx2[j] with weight
    w1 w2 (a pure pointer chase)."""
    rng = np.random.default_rng(3)
    idx1, w1 = cases.edges(rng, 2, 50, 3, 1)
    idx2, w2 = cases.edges(rng, 2, 50, 3, 1)
    for s1 in (1, 3):
        io, wo = orc.ser_forward(idx1, w1, idx2, w2, s1=s1)
        b, i, h = np.meshgrid(np.arange(2), np.arange(50), np.arange(3), indexing="ij")
        j = idx1[..., 0]
        np.testing.assert_array_equal(io[..., 0], idx2[b, j, h, 0])
        np.testing.assert_array_equal(
            wo[..., 0], (w1[..., 0].astype(np.float64) * w2[b, j, h, 0]).astype(np.float32))
        assert (io[..., 1:] == 0).all() and (wo[..., 1:] == 0).all()


def test_ser_forward_self_loops_closed_form(orc):
    """Every edge points at its own token: all s2 s3 paths end at i, so A'
    row i is (i, (sum w1)(sum w2)) followed by padding."""
    rng = np.random.default_rng(4)
    n, s = 40, 3
    idx = np.broadcast_to(np.arange(n).reshape(1, n, 1, 1), (1, n, 2, s)).astype(np.int32)
    w1 = (rng.random((1, n, 2, s)) + 0.1).astype(np.float32)
    w2 = (rng.random((1, n, 2, s)) + 0.1).astype(np.float32)
    io, wo, we = orc.ser_forward(idx, w1, idx, w2, s1=4, exact=True)
    np.testing.assert_array_equal(io[..., 0], idx[..., 0])
    prod = w1.astype(np.float64).sum(-1) * w2.astype(np.float64).sum(-1)
    np.testing.assert_allclose(we[..., 0], prod, rtol=1e-15)
    assert (io[..., 1:] == 0).all() and (wo[..., 1:] == 0).all()


def test_ser_forward_invariants(orc):
    """Causality survives composition (idx' <= i), weights stay >= 0, kept
    targets are distinct, padding is exactly (0, 0), slots are ordered, and
    the kept mass is at most sum_a w1 * max_j sum_c w2."""
    idx, w = synth.edges(11, B=2, n=300, hkv=2, s=4, mode="mixed")
    io, wo, we = orc.ser_forward(idx, w, idx, w, s1=4, exact=True)
    i = np.arange(300).reshape(1, 300, 1, 1)
    assert (io <= i).all() and (io >= 0).all() and (wo >= 0).all()
    pad = wo == 0
    assert (io[pad] == 0).all()
    assert (np.diff(wo, axis=-1) <= 0).all()
    for b, n_, h in np.ndindex(2, 300, 2):
        live = io[b, n_, h][~pad[b, n_, h]]
        assert len(set(live.tolist())) == len(live)
    rowmass = w.astype(np.float64).sum(-1)
    bound = rowmass * rowmass.max(axis=1, keepdims=True)
    assert (we.sum(-1) <= bound * (1 + 1e-12)).all()


# --------------------------------------------------------------- SER backward
def _ser_case(rng, n=30, s=3, s1=3, ties=False, pad=0.15):
    idx1, w1 = cases.edges(rng, 1, n, 2, s, pad_frac=pad, ties=ties)
    idx2, w2 = cases.edges(rng, 1, n, 2, s, pad_frac=pad, ties=ties)
    return idx1, w1, idx2, w2, s1


def test_ser_backward_matches_dense(orc):
    rng = np.random.default_rng(21)
    for case in range(40):
        idx1, w1, idx2, w2, s1 = _ser_case(rng, n=int(rng.integers(2, 40)),
                                           s=int(rng.integers(1, 5)), s1=int(rng.integers(1, 5)))
        io, wo = orc.ser_forward(idx1, w1, idx2, w2, s1=s1)
        dwo = rng.standard_normal(io.shape)
        dw1, dw2 = orc.ser_backward(idx1, w1, idx2, w2, io, wo, dwo)
        r1, r2 = dense_ref.ser_backward(idx1, w1, idx2, w2, io, wo, dwo)
        np.testing.assert_allclose(dw1, r1, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dw2, r2, rtol=1e-12, atol=1e-14)


def test_ser_backward_aliased_legs_sum(orc):
    """A' = Sparsify(A A): the gradient of A is dw1 + dw2 of distinct legs."""
    idx, w = synth.edges(5, B=1, n=80, hkv=2, s=4, mode="mixed")
    io, wo = orc.ser_forward(idx, w, idx, w, s1=4)
    dwo = np.random.default_rng(6).standard_normal(io.shape)
    a1, a2 = orc.ser_backward(idx, w, idx, w, io, wo, dwo, aliased=True)
    d1, d2 = orc.ser_backward(idx, w, idx, w, io, wo, dwo)
    assert a1 is a2
    np.testing.assert_allclose(a1, d1 + d2, rtol=1e-13, atol=1e-15)


def test_ser_backward_finite_differences(orc):
    """Central differences of L = sum_t dw'_t w'_t (unrounded double) in w1, w2
    at fixed selection."""
    rng = np.random.default_rng(8)
    idx1, w1, idx2, w2, s1 = _ser_case(rng, n=16, s=3, s1=3, pad=0.1)
    w1 = w1.astype(np.float64); w2 = w2.astype(np.float64)
    io, wo = orc.ser_forward(idx1, w1, idx2, w2, s1=s1)
    dwo = rng.standard_normal(io.shape)
    dw1, dw2 = orc.ser_backward(idx1, w1, idx2, w2, io, wo, dwo)

    def loss(a, b):
        jo, _, we = orc.ser_forward(idx1, a, idx2, b, s1=s1, exact=True)
        return float((dwo * we).sum()), jo

    checked = 0
    for which, arr, grad in (("w1", w1, dw1), ("w2", w2, dw2)):
        for flat in rng.choice(arr.size, size=40, replace=False):
            pos = np.unravel_index(flat, arr.shape)
            if arr[pos] <= 0:
                assert grad[pos] == 0.0
                continue
            eps = 1e-6 * arr[pos]
            ap, am = arr.copy(), arr.copy()
            ap[pos] += eps; am[pos] -= eps
            if which == "w1":
                (lp, jp), (lm, jm) = loss(ap, w2), loss(am, w2)
            else:
                (lp, jp), (lm, jm) = loss(w1, ap), loss(w1, am)
            if not ((jp == io).all() and (jm == io).all()):
                continue                                   # selection moved
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (which, pos, fd, grad[pos])
            checked += 1
    assert checked >= 40


def test_ser_backward_euler_identities(orc):
    """w' is homogeneous of degree 1 in the leg-1 row and in A2, so
    sum_a w1 dw1 = sum_t w' dw' per unit, and sum w2 dw2 = sum w' dw' overall."""
    rng = np.random.default_rng(9)
    idx1, w1, idx2, w2, s1 = _ser_case(rng, n=60, s=4, s1=3, pad=0.1)
    io, wo, we = orc.ser_forward(idx1, w1, idx2, w2, s1=s1, exact=True)
    dwo = rng.standard_normal(io.shape)
    dw1, dw2 = orc.ser_backward(idx1, w1, idx2, w2, io, wo, dwo)
    lhs = (w1.astype(np.float64) * dw1).sum(-1)
    rhs = (we * dwo).sum(-1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose((w2.astype(np.float64) * dw2).sum(), rhs.sum(), rtol=1e-12)


# ---------------------------------------------------------------- SEA forward
def _sea_case(rng, B=1, n=24, hq=4, hkv=2, d=8, s=3, pad=0.0, ties=False, dead=0.0):
    q = rng.standard_normal((B, n, hq, d)); k = rng.standard_normal((B, n, hkv, d))
    v = rng.standard_normal((B, n, hkv, d)); do = rng.standard_normal((B, n, hq, d))
    idx, w = cases.edges(rng, B, n, hkv, s, pad_frac=pad, ties=ties, dead_frac=dead)
    return q, k, v, idx, w, do


def test_sea_forward_backward_match_dense(orc):
    rng = np.random.default_rng(31)
    for case in range(60):
        hkv = int(rng.integers(1, 3)); G = int(rng.integers(1, 4))
        q, k, v, idx, w, do = _sea_case(
            rng, B=int(rng.integers(1, 3)), n=int(rng.integers(1, 30)), hq=hkv * G, hkv=hkv,
            d=int(rng.choice([4, 8, 16])), s=int(rng.integers(1, 6)),
            pad=0.25 * (case % 3 == 0), ties=bool(case % 2), dead=0.2 * (case % 4 == 0))
        o = orc.sea_forward(q, k, v, idx, w)
        dq, dk, dv, dw = orc.sea_backward(q, k, v, idx, w, do)
        ro, rdq, rdk, rdv, rdw = dense_ref.sea(q, k, v, idx, w, do)
        for a, b_ in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv), (dw, rdw)):
            np.testing.assert_allclose(a, b_, rtol=1e-10, atol=1e-12)


def test_sea_slot_probabilities_match_dense(orc):
    """The per-slot probabilities the oracle reports: summed over the slots
    that share a target they are the dense attention probabilities, dead
    slots get 0, and they rebuild the output o = sum_t p_t v[idx_t]."""
    rng = np.random.default_rng(37)
    for case in range(30):
        hkv = int(rng.integers(1, 3)); G = int(rng.integers(1, 4))
        B, n, s = int(rng.integers(1, 3)), int(rng.integers(1, 25)), int(rng.integers(1, 6))
        q, k, v, idx, w, _ = _sea_case(rng, B=B, n=n, hq=hkv * G, hkv=hkv, d=8, s=s,
                                       pad=0.25 * (case % 3 == 0), ties=bool(case % 2),
                                       dead=0.2 * (case % 4 == 0))
        o, p = orc.sea_forward(q, k, v, idx, w, probs=True)
        P = dense_ref.sea_probs(q, k, idx, w)
        live = np.repeat(w > 0, G, axis=2)                  # [B, n, hq, s]
        assert (p[~live] == 0).all()
        tgt = np.repeat(idx, G, axis=2)
        for b in range(B):
            for i in range(n):
                for hh in range(hkv * G):
                    acc = {}
                    for t in range(s):
                        if live[b, i, hh, t]:
                            acc[tgt[b, i, hh, t]] = acc.get(tgt[b, i, hh, t], 0.0) + p[b, i, hh, t]
                    for j, pj in acc.items():
                        assert abs(pj - P[b, hh, i, j]) <= 1e-12, (case, b, i, hh, j)
        vg = v[np.arange(B)[:, None, None, None], idx, np.arange(hkv)[None, None, :, None]]
        ob = np.einsum("bnhgt,bnhtd->bnhgd", p.reshape(B, n, hkv, G, s), vg)
        np.testing.assert_allclose(ob.reshape(o.shape), o, rtol=1e-12, atol=1e-12)


def test_sea_tiny_config_dense(orc):
    p = synth.PRESETS["tiny"]
    idx, w = synth.edges(p.seed, p.B, p.n, p.hkv, p.s1, mode=p.mode)
    q = synth.normal(p.seed, "q", (p.B, p.n, p.hq, p.d)).numpy()
    k = synth.normal(p.seed, "k", (p.B, p.n, p.hkv, p.d)).numpy()
    v = synth.normal(p.seed, "v", (p.B, p.n, p.hkv, p.d)).numpy()
    do = synth.normal(p.seed, "dout", (p.B, p.n, p.hq, p.d)).numpy()
    o = orc.sea_forward(q, k, v, idx, w)
    grads = orc.sea_backward(q, k, v, idx, w, do)
    ref = dense_ref.sea(q, k, v, idx, w, do)
    for a, b_ in zip((o,) + grads, ref):
        np.testing.assert_allclose(a, b_, rtol=1e-10, atol=1e-12)


def test_sea_single_slot_closed_form(orc):
    """s1 = 1: the softmax has one term, so o = v[idx], dq = dk = dw = 0 and
    dv[idx] collects the upstream gradients of every query head of the group."""
    rng = np.random.default_rng(41)
    q, k, v, idx, w, do = _sea_case(rng, B=2, n=20, hq=6, hkv=2, d=8, s=1)
    o = orc.sea_forward(q, k, v, idx, w)
    dq, dk, dv, dw = orc.sea_backward(q, k, v, idx, w, do)
    b, i, h = np.meshgrid(np.arange(2), np.arange(20), np.arange(2), indexing="ij")
    gathered = v[b, idx[..., 0], h]                              # [B,n,hkv,d]
    np.testing.assert_allclose(o.reshape(2, 20, 2, 3, 8), gathered[:, :, :, None, :] *
                               np.ones((1, 1, 1, 3, 1)), rtol=1e-15)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0 and np.abs(dw).max() == 0
    ref_dv = np.zeros_like(v)
    dsum = do.reshape(2, 20, 2, 3, 8).sum(3)
    for bb, ii, hh in np.ndindex(2, 20, 2):
        ref_dv[bb, idx[bb, ii, hh, 0], hh] += dsum[bb, ii, hh]
    np.testing.assert_allclose(dv, ref_dv, rtol=1e-14, atol=1e-14)


def test_sea_zero_query_closed_form(orc):
    """q = 0: every node expert is equal, so p_t = w_t / sum w and
    o = sum_t w_t v[idx_t] / sum_t w_t."""
    rng = np.random.default_rng(42)
    q, k, v, idx, w, _ = _sea_case(rng, B=1, n=30, hq=4, hkv=2, d=8, s=4, pad=0.2)
    q[:] = 0
    o = orc.sea_forward(q, k, v, idx, w)
    wd = w.astype(np.float64)
    num = np.zeros((1, 30, 2, 8))
    for i, h, t in np.ndindex(30, 2, 4):
        num[0, i, h] += wd[0, i, h, t] * v[0, idx[0, i, h, t], h]
    den = wd.sum(-1)
    ref = np.where(den[..., None] > 0, num / np.where(den > 0, den, 1)[..., None], 0)
    np.testing.assert_allclose(o.reshape(1, 30, 2, 2, 8), ref[:, :, :, None, :].repeat(2, 3),
                               rtol=1e-13, atol=1e-14)


def test_sea_constant_values_and_conservation(orc):
    """Probabilities sum to one (constant v rows give o = v), and per
    (b, h): sum_j dv[j] = sum of dout over live rows and heads,
    sum_j dk[j] = 0, and per unit sum_t w_t dw_t = 0 (SEA is invariant to
    scaling a row of w)."""
    rng = np.random.default_rng(43)
    q, k, v, idx, w, do = _sea_case(rng, B=2, n=40, hq=4, hkv=2, d=8, s=4, pad=0.2)
    vc = np.broadcast_to(rng.standard_normal((2, 1, 2, 8)), v.shape).copy()
    o = orc.sea_forward(q, k, vc, idx, w)
    live = (w > 0).any(-1)                                        # [B,n,hkv]
    exp = np.where(live[..., None, None], vc[:, :, :, None, :], 0.0)
    np.testing.assert_allclose(o.reshape(2, 40, 2, 2, 8), exp.repeat(2, 3), rtol=1e-13, atol=1e-14)
    dq, dk, dv, dw = orc.sea_backward(q, k, v, idx, w, do)
    dsum = (do.reshape(2, 40, 2, 2, 8).sum(3) * live[..., None]).sum(1)
    np.testing.assert_allclose(dv.sum(1), dsum, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk.sum(1), 0.0, atol=1e-12)
    np.testing.assert_allclose((w * dw).sum(-1), 0.0, atol=1e-12)


def test_sea_finite_differences(orc):
    """Central differences of L = sum dout . o in q, k, v and w."""
    rng = np.random.default_rng(44)
    q, k, v, idx, w, do = _sea_case(rng, B=1, n=10, hq=4, hkv=2, d=4, s=3, pad=0.15)
    w = w.astype(np.float64)
    grads = orc.sea_backward(q, k, v, idx, w, do)
    names = ("q", "k", "v", "w")
    base = dict(q=q, k=k, v=v, w=w)
    gmap = dict(q=grads[0], k=grads[1], v=grads[2], w=grads[3])

    def loss(**kw):
        a = dict(base); a.update(kw)
        return float((do * orc.sea_forward(a["q"], a["k"], a["v"], idx, a["w"])).sum())

    for name in names:
        arr = base[name]
        for flat in rng.choice(arr.size, size=min(arr.size, 25), replace=False):
            pos = np.unravel_index(flat, arr.shape)
            if name == "w" and arr[pos] <= 0:
                assert gmap["w"][pos] == 0.0
                continue
            eps = 1e-6 * max(1.0, abs(arr[pos])) if name != "w" else 1e-6 * arr[pos]
            ap, am = arr.copy(), arr.copy()
            ap[pos] += eps; am[pos] -= eps
            fd = (loss(**{name: ap}) - loss(**{name: am})) / (2 * eps)
            assert abs(fd - gmap[name][pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd,
                                                                        gmap[name][pos])


def test_sea_all_padding_row_is_zero(orc):
    rng = np.random.default_rng(45)
    q, k, v, idx, w, do = _sea_case(rng, B=1, n=8, hq=2, hkv=1, d=4, s=2)
    idx[0, 5] = 0; w[0, 5] = 0
    o = orc.sea_forward(q, k, v, idx, w)
    dq, dk, dv, dw = orc.sea_backward(q, k, v, idx, w, do)
    assert (o[0, 5] == 0).all() and (dq[0, 5] == 0).all() and (dw[0, 5] == 0).all()


# ------------------------------------------------------ printed KV-access figures
def test_kv_access_fraction_matches_printed_values(orc):
    """The page prints SEA's KV access at n = 4096 as 0.098% (2 edges per KV
    head) and 0.195% (4) of dense causal attention, which reads (n+1)/2
    positions per query on average.  Count the rows the oracle reads."""
    with open(os.path.join(GOLDEN, "kv_access.json")) as f:
        g = json.load(f)
    n = g["n"]
    for s, printed in zip(g["retrieved_per_kv_head"], g["percent_of_dense_causal"]):
        idx, w = synth.edges(99, 1, n, 1, s, mode="mixed")
        q = np.zeros((1, n, 1, 4)); kv = np.zeros((1, n, 1, 4))
        _, rows = orc.sea_forward(q, kv, kv, idx, w, count=True)
        per_query = rows / n
        assert per_query == s
        assert round(100 * per_query / ((n + 1) / 2), 3) == printed


# ------------------------------------------------------ leg construction
def _leg_case(rng, B, n, hkv, K, ties=False, pad=0.0, dead=0.0, zero_alpha=0.0):
    idx, w = cases.edges(rng, B, n, hkv, K, pad_frac=pad, ties=ties, dead_frac=dead)
    alpha = (rng.choice(cases.TIE_WEIGHTS, size=(hkv, K)) if ties
             else rng.random((hkv, K)) + 0.05)
    if zero_alpha:
        alpha = np.where(rng.random(alpha.shape) < zero_alpha, 0.0, alpha)
    return idx, w, alpha.astype(np.float32).astype(np.float64)


def test_leg_mix_matches_dense_mixture(orc):
    """Leg construction against dense rows sum_k alpha_k w_k e_{idx_k}, top-s:
    random shapes, padding, dead slots, zero mixing weights, duplicates and
    exact ties (dyadic weights)."""
    rng = np.random.default_rng(2024)
    for case in range(300):
        B, hkv = (int(x) for x in rng.integers(1, 3, size=2))
        n, K, s = int(rng.integers(1, 20)), int(rng.integers(1, 12)), int(rng.integers(1, 6))
        idx, w, alpha = _leg_case(rng, B, n, hkv, K, ties=bool(case % 2),
                                  pad=0.2 * (case % 3 == 0), dead=0.2 * (case % 5 == 0),
                                  zero_alpha=0.2 * (case % 4 == 0))
        io, wo = orc.leg_mix_forward(idx, w, alpha, s)
        ref_io, ref_wo, kth, nxt = dense_ref.leg_mix(idx, w, alpha, s)
        assert_ser_equal(io, wo, ref_io, ref_wo, kth, nxt)


def test_leg_mix_single_slot_closed_form(orc):
    """K = 1: the leg is the stored edge with weight alpha * w when positive,
    else padding."""
    rng = np.random.default_rng(5)
    idx, w, alpha = _leg_case(rng, 2, 15, 3, 1, dead=0.3, zero_alpha=0.3)
    io, wo = orc.leg_mix_forward(idx, w, alpha, 2)
    prod = (w[..., 0].astype(np.float64) * alpha[None, None, :, 0]).astype(np.float32)
    live = prod > 0
    np.testing.assert_array_equal(io[..., 0], np.where(live, idx[..., 0], 0))
    np.testing.assert_array_equal(wo[..., 0], np.where(live, prod, 0.0))
    assert (io[..., 1] == 0).all() and (wo[..., 1] == 0).all()


def test_leg_mix_backward_matches_dense_and_differences(orc):
    """Backward against the dense mixture's chain rule, and central
    differences of the kept weight sum (selection fixed, no near ties)."""
    rng = np.random.default_rng(99)
    for case in range(40):
        B, hkv, n, K, s = 1, 2, int(rng.integers(2, 14)), int(rng.integers(1, 9)), 3
        idx, w, alpha = _leg_case(rng, B, n, hkv, K, pad=0.1, dead=0.1, zero_alpha=0.1)
        io, wo = orc.leg_mix_forward(idx, w, alpha, s)
        dleg = rng.standard_normal(io.shape)
        dw, da = orc.leg_mix_backward(idx, w, alpha, io, wo, dleg)
        rdw, rda = dense_ref.leg_mix_backward(idx, w, alpha, io, wo, dleg)
        np.testing.assert_allclose(dw, rdw, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(da, rda, rtol=1e-12, atol=1e-14)
    # central differences of f = sum_t dleg_t * (exact kept weight of slot t)
    rng = np.random.default_rng(7)
    idx, w, alpha = _leg_case(rng, 1, 10, 2, 6)
    io, wo = orc.leg_mix_forward(idx, w, alpha, 3)
    dleg = rng.standard_normal(io.shape)
    dw, da = orc.leg_mix_backward(idx, w, alpha, io, wo, dleg)

    def f(w_, a_):
        tot = 0.0
        for b in range(1):
            for i in range(10):
                for h in range(2):
                    for t in range(3):
                        if wo[b, i, h, t] > 0:
                            m = io[b, i, h, t]
                            sel = idx[b, i, h] == m
                            tot += dleg[b, i, h, t] * float((w_[b, i, h] * a_[h])[sel].sum())
        return tot
    eps = 1e-6
    wd = w.astype(np.float64)
    for (b, i, h, k) in [(0, 3, 0, 1), (0, 9, 1, 5), (0, 6, 1, 0)]:
        if wd[b, i, h, k] <= 0:
            continue
        p, m = wd.copy(), wd.copy()
        p[b, i, h, k] += eps; m[b, i, h, k] -= eps
        assert abs((f(p, alpha) - f(m, alpha)) / (2 * eps) - dw[b, i, h, k]) < 1e-6
    for (h, k) in [(0, 2), (1, 4)]:
        p, m = alpha.copy(), alpha.copy()
        p[h, k] += eps; m[h, k] -= eps
        assert abs((f(wd, p) - f(wd, m)) / (2 * eps) - da[h, k]) < 1e-6


# --------------------------------------------------------- refresh edges
def test_dense_refresh_matches_dense_attention(orc):
    """Refresh edges against dense causal attention (tests/dense_ref.py with
    every earlier position an edge of weight 1): the per-head log-sum-exp,
    and the group-mean probabilities of the kept positions, which must be
    the s largest (equal values to the lower index)."""
    rng = np.random.default_rng(11)
    for case in range(12):
        hkv, G = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        B, n, d, s = 1 + case % 2, int(rng.integers(1, 30)), 8, int(rng.integers(1, 6))
        q = rng.standard_normal((B, n, hkv * G, d))
        k = rng.standard_normal((B, n, hkv, d))
        if case % 3 == 0:
            q[:, :, :, :] = np.round(q * 2) / 2           # repeated scores: ties
            k[:, :, :, :] = np.round(k * 2) / 2
        io, wo, lse = orc.dense_refresh(q, k, s)
        full = np.broadcast_to(np.arange(n).reshape(1, n, 1, 1), (B, n, hkv, n)).copy()
        full = np.minimum(full, np.arange(n).reshape(1, 1, 1, n)).astype(np.int32)
        wfull = (np.arange(n).reshape(1, 1, 1, n) <= np.arange(n).reshape(1, n, 1, 1))
        wfull = np.broadcast_to(wfull, (B, n, hkv, n)).astype(np.float32)
        P = dense_ref.sea_probs(q, k, full, wfull)          # [B, hq, n, n]
        pbar = P.reshape(B, hkv, G, n, n).mean(axis=2)       # [B, hkv, n, n]
        scores = np.einsum("bihd,bjhd->bhij", q, np.repeat(k, G, axis=2)) / np.sqrt(d)
        mask = np.tril(np.ones((n, n), bool))
        ref_lse = np.log(np.where(mask, np.exp(scores), 0.0).sum(-1))
        np.testing.assert_allclose(lse, ref_lse.transpose(0, 2, 1), rtol=1e-12, atol=1e-12)
        for b in range(B):
            for i in range(n):
                for h in range(hkv):
                    assert_valid_top(io[b, i, h], wo[b, i, h], pbar[b, h, i, :i + 1], s)


def assert_valid_top(idx, w, row, s, rel=1e-9):
    """idx/w is the top-s of ``row`` (values desc, equal values to the lower
    index), with values equal when they agree within ``rel`` (the reference
    rounds its sums differently)."""
    m = min(s, len(row))
    order = np.argsort(-row, kind="stable")
    kth = row[order[m - 1]]
    tol = rel * max(float(row.max()), 1e-300)
    picked = idx[:m]
    assert len(set(picked.tolist())) == m, picked
    assert (row[picked] >= kth - tol).all(), (picked, row[picked], kth)
    for a, b_ in zip(picked[:-1], picked[1:]):
        va, vb = row[a], row[b_]
        assert va >= vb - tol, (picked, row[picked])
        if abs(va - vb) <= tol:
            assert a < b_, (picked, row[picked])
    np.testing.assert_allclose(w[:m], row[picked].astype(np.float32), rtol=1e-6)
    assert (idx[m:] == 0).all() and (w[m:] == 0).all()
