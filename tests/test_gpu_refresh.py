"""GPU parity of the refresh edges (gm_dense_refresh) against the oracle.

The kernel forms the scores in fp32 from bf16 products on the matrix cores;
the oracle in fp64 from the same bf16 values.  The bars, from that
arithmetic:

* lse within 2e-4 absolute.  Each product of two bf16 values is exact in
  fp32; a dot of d of them rounds to at most d * 2^-24 * sum|q_c k_c|
  (< 1e-3 for d = 256 and these N(0, 1) or 3 x N(0, 1) draws), times the
  scale 1/sqrt(d), plus a few ulps from exp2/log2.  In practice ~1e-6.
* The kept positions as a valid top-s: the oracle is run for s + 8
  positions; every position the kernel keeps is among them, its weight
  within 1e-3 relative (+1e-7 absolute) of the oracle's pbar (an error e in
  an exponent is a relative error e in the probability), no position left
  out beats a kept one by more than that, the list is sorted by weight with
  exact ties to the lower position, and slots past the i+1 positions of
  token i hold (0, 0).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_dynamic_routing_amd as gm
import synth
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

LSE_TOL = 2e-4
W_REL, W_ABS = 1e-3, 1e-7


def check_rows(gi, gw, oi, ow, s):
    """gi/gw [B, n, hkv, s] from the kernel, oi/ow [B, n, hkv, s + 8] from
    the oracle."""
    B, n, hkv, _ = gi.shape
    bad = 0
    for b in range(B):
        for i in range(n):
            m = min(s, i + 1)
            for h in range(hkv):
                pick, w = gi[b, i, h], gw[b, i, h]
                try:
                    assert (pick[m:] == 0).all() and (w[m:] == 0).all(), "padding"
                    pk, wk = pick[:m], w[:m]
                    assert len(set(pk.tolist())) == m, "repeated position"
                    assert (pk >= 0).all() and (pk <= i).all(), "position out of range"
                    assert (wk > 0).all() and (np.diff(wk) <= 0).all(), "weights not sorted"
                    for a in range(m - 1):
                        if wk[a] == wk[a + 1]:
                            assert pk[a] < pk[a + 1], "exact tie not to the lower position"
                    mo = min(oi.shape[-1], i + 1)
                    ref = dict(zip(oi[b, i, h, :mo].tolist(), ow[b, i, h, :mo].tolist()))
                    for j, wj in zip(pk.tolist(), wk.tolist()):
                        assert j in ref, f"position {j} outside the oracle's top {mo}"
                        assert abs(wj - ref[j]) <= W_REL * ref[j] + W_ABS, \
                            f"weight {wj} vs {ref[j]} at {j}"
                    kth = min(ref[j] for j in pk.tolist())
                    for j, v in ref.items():
                        if j not in pk:
                            assert v <= kth * (1 + W_REL) + W_ABS, f"left out {j} ({v} > {kth})"
                except AssertionError as e:
                    bad += 1
                    if bad <= 3:
                        say(f"    row b={b} i={i} h={h}: {e}; kernel {pick} {w}; "
                            f"oracle {oi[b, i, h]} {ow[b, i, h]}")
    assert bad == 0, f"{bad} rows fail"


REFRESH_CASES = [
    # B, n, hkv, G, d, s, score scale, seed
    (2, 300, 2, 2, 128, 4, 1.0, 1),      # the measured shape's head layout, ragged tail
    (1, 129, 2, 2, 128, 4, 3.0, 2),      # peaky attention; a last tile of one token
    (2, 200, 1, 8, 64, 8, 1.0, 3),       # widest group; the most kept positions
    (1, 260, 2, 2, 256, 1, 2.0, 4),      # d = 256, top-1
    (3, 97, 3, 1, 128, 2, 1.0, 5),       # one head per group, less than one tile
    (1, 517, 1, 4, 64, 4, 3.0, 6),       # several key tiles, G = 4
    (2, 130, 2, 4, 128, 3, 1.0, 7),      # s not a power of two
    (1, 300, 1, 2, 256, 8, 2.0, 13),     # d = 256 with the longest list (registers spill)
    (2, 1000, 3, 1, 64, 5, 3.0, 14),     # three KV heads (pairs not a power of two), 4 tiles
    (1, 300, 2, 1, 256, 8, 2.0, 15),     # one pass (G = 1) at d = 256, the longest list
    (2, 700, 2, 1, 128, 4, 0.3, 16),     # one pass, flat attention (many near-equal scores)
]


def _inputs(B, n, hkv, G, d, amp, seed):
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((B, n, hkv * G, d), dtype=np.float32) * amp)
    k = torch.from_numpy(rng.standard_normal((B, n, hkv, d), dtype=np.float32))
    return q.to(torch.bfloat16), k.to(torch.bfloat16)


@pytest.mark.parametrize("B,n,hkv,G,d,s,amp,seed", REFRESH_CASES,
                         ids=[f"B{c[0]}-n{c[1]}-hkv{c[2]}-G{c[3]}-d{c[4]}-s{c[5]}"
                              for c in REFRESH_CASES])
def test_refresh_matches_oracle(B, n, hkv, G, d, s, amp, seed):
    say(f"case refresh B={B} n={n} hkv={hkv} G={G} d={d} s={s} amp={amp}")
    q, k = _inputs(B, n, hkv, G, d, amp, seed)
    io, wo, lse = gm.dense_refresh(dev(q), dev(k), s)
    torch.cuda.synchronize()
    oi, ow, olse = oracle.get().dense_refresh(q, k, s + 8)
    err = float(np.abs(host(lse) - olse).max())
    say(f"    lse max error {err:.3e} (bar {LSE_TOL:g})")
    assert err <= LSE_TOL
    check_rows(host(io), host(wo), oi, ow, s)


def test_refresh_with_the_layers_own_lse():
    """lse given: only the selection runs, lse is left as passed."""
    B, n, hkv, G, d, s = 2, 300, 2, 2, 128, 4
    q, k = _inputs(B, n, hkv, G, d, 2.0, 8)
    oi, ow, olse = oracle.get().dense_refresh(q, k, s + 8)
    lse = dev(torch.from_numpy(olse.astype(np.float32)))
    before = lse.clone()
    io, wo, lse2 = gm.dense_refresh(dev(q), dev(k), s, lse=lse)
    torch.cuda.synchronize()
    assert lse2 is lse and torch.equal(lse, before)
    check_rows(host(io), host(wo), oi, ow, s)


def test_refresh_tiny_sequences_pad():
    """n < s: token i keeps its i+1 positions, the rest are (0, 0); n = 1
    keeps (0, 1)."""
    for n, s in ((1, 4), (2, 8), (3, 4)):
        q, k = _inputs(2, n, 2, 2, 64, 1.0, 9 + n)
        io, wo, lse = gm.dense_refresh(dev(q), dev(k), s)
        torch.cuda.synchronize()
        oi, ow, olse = oracle.get().dense_refresh(q, k, s)
        assert float(np.abs(host(lse) - olse).max()) <= LSE_TOL
        check_rows(host(io), host(wo), oi, ow, s)
        gi = host(io)
        assert (gi[:, 0, :, 0] == 0).all()
        np.testing.assert_allclose(host(wo)[:, 0, :, 0], 1.0, rtol=1e-6)


@pytest.mark.parametrize("G", [2, 1])
def test_refresh_repeated_keys_tie_to_the_lower_position(G):
    """Equal key rows give equal probabilities: the lower position is kept
    first (both sides compute the two scores the same way; G = 1 takes the
    one-pass kernel, which ranks by the raw score)."""
    B, n, hkv, d, s = 1, 200, 2, 128, 4
    q, k = _inputs(B, n, hkv, G, d, 3.0, 12)
    k[:, 1::2] = k[:, 0::2][:, : k[:, 1::2].shape[1]]   # position 2t+1 repeats 2t
    io, wo, lse = gm.dense_refresh(dev(q), dev(k), s)
    torch.cuda.synchronize()
    oi, ow, _ = oracle.get().dense_refresh(q, k, s + 8)
    check_rows(host(io), host(wo), oi, ow, s)
    gi, gw = host(io), host(wo)
    pairs = 0
    for i in range(1, n):
        for h in range(hkv):
            for a in range(s - 1):
                if gw[0, i, h, a] == gw[0, i, h, a + 1] and gw[0, i, h, a] > 0:
                    assert gi[0, i, h, a] < gi[0, i, h, a + 1]
                    pairs += 1
    say(f"    exact ties seen: {pairs}")
    assert pairs > 0


def test_refresh_full_size_pairs():
    """The dense layer of the measured model (B=8, n=4096, 16 query / 8 KV
    heads, d=128, s=4): every row of two (batch, KV head) pairs against the
    oracle run on those pairs alone, and properties that hold for all rows."""
    B, n, hq, hkv, d, s = 8, 4096, 16, 8, 128, 4
    G = hq // hkv
    seed = synth.BASE_SEED + 40
    q = synth.normal(seed, "q", (B, n, hq, d), torch.bfloat16)
    k = synth.normal(seed, "k", (B, n, hkv, d), torch.bfloat16)
    say(f"case refresh full size B={B} n={n} hq={hq} hkv={hkv} d={d} s={s}")
    io, wo, lse = gm.dense_refresh(dev(q), dev(k), s)
    torch.cuda.synchronize()
    gi, gw, gl = host(io), host(wo), host(lse)
    # every row: positions causal and distinct, weights sorted and summing <= 1
    pos = np.arange(n).reshape(1, n, 1, 1)
    m = np.minimum(s, pos + 1)
    slot = np.arange(s).reshape(1, 1, 1, s)
    live = np.broadcast_to(slot < m, gw.shape)
    assert ((gi <= pos) & (gi >= 0)).all()
    assert (gw[live] > 0).all() and (gw[~live] == 0).all() and (gi[~live] == 0).all()
    assert (np.diff(gw, axis=-1) <= 0).all()
    assert (gw.sum(-1) <= 1 + 1e-5).all()
    srt = np.sort(np.where(live, gi, -1 - np.broadcast_to(slot, gi.shape)), axis=-1)
    assert (np.diff(srt, axis=-1) != 0).all()
    assert np.isfinite(gl).all()
    for b, h in ((0, 0), (B - 1, hkv - 1)):
        qp = q[b:b + 1, :, h * G:(h + 1) * G].contiguous()
        kp = k[b:b + 1, :, h:h + 1].contiguous()
        oi, ow, olse = oracle.get().dense_refresh(qp, kp, s + 8)
        err = float(np.abs(gl[b:b + 1, :, h * G:(h + 1) * G] - olse).max())
        say(f"    pair ({b}, {h}): lse max error {err:.3e}")
        assert err <= LSE_TOL
        check_rows(gi[b:b + 1, :, h:h + 1], gw[b:b + 1, :, h:h + 1], oi, ow, s)
