"""GPU parity over shapes, dtypes and the degenerate cases of the method,
through the C ABI, against the oracle on every output element.

Sizes are small (the oracle finishes in well under a second) but span
several workgroups and a ragged tail (token counts that are not a multiple
of the units per workgroup).
"""
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

SEA_SHAPES = [
    # dtype, d, G, s, n
    (torch.bfloat16, 128, 2, 4, 67),    # the measured layer's geometry
    (torch.bfloat16, 128, 2, 4, 64),    # segments of 32 tokens: saved records read as blocks
    (torch.bfloat16, 128, 2, 2, 67),    # retrieving 2 per KV head
    (torch.bfloat16, 128, 1, 3, 45),    # slot count not a power of two
    (torch.bfloat16, 128, 4, 8, 33),    # two slot chunks per unit
    (torch.bfloat16, 128, 2, 5, 33),    # ragged second chunk
    (torch.bfloat16, 64, 8, 4, 40),     # 128-byte rows: low half of each lane's registers
    (torch.bfloat16, 64, 1, 2, 29),
    (torch.bfloat16, 64, 16, 1, 21),
    (torch.float32, 32, 2, 4, 33),      # 128-byte fp32 rows (forward row kernel)
    (torch.bfloat16, 256, 2, 4, 29),    # 32 lanes per row; forward: two pieces per lane
    (torch.bfloat16, 256, 1, 1, 31),    # 512-byte rows, one slot
    (torch.bfloat16, 256, 8, 2, 23),    # 512-byte rows, two query chunks
    (torch.bfloat16, 16, 16, 6, 50),    # 2 lanes per row, many units per wave
    (torch.bfloat16, 32, 2, 64, 21),    # the widest slot count
    (torch.float32, 16, 2, 2, 64),      # the tiny preset's geometry
    (torch.float32, 128, 2, 4, 37),
    (torch.float32, 128, 16, 3, 19),    # 512-byte fp32 rows, four query chunks
    (torch.float32, 256, 1, 3, 19),     # 64 lanes per row: one slot per chunk
    (torch.float32, 32, 4, 9, 41),
    (torch.float32, 64, 2, 4, 37),      # fp32 rows of 256 bytes (fp64 arithmetic)
    (torch.float32, 64, 4, 1, 26),
    (torch.bfloat16, 128, 16, 1, 23),   # one slot, sixteen query heads
    (torch.bfloat16, 128, 8, 2, 45),
    (torch.bfloat16, 128, 2, 4, 1),     # fewer units than XCDs
    # group sizes other than powers of two (the general kernels)
    (torch.bfloat16, 128, 3, 4, 41),
    (torch.bfloat16, 128, 6, 2, 37),
    (torch.bfloat16, 64, 12, 4, 23),
    (torch.float32, 64, 3, 4, 33),
    (torch.float32, 128, 6, 3, 29),
    (torch.bfloat16, 256, 5, 3, 19),
    # groups wider than the row kernels' sixteen heads (multi-query widths)
    (torch.bfloat16, 64, 32, 4, 29),
    (torch.float32, 32, 24, 2, 21),
]


def _sea_inputs(rng, dtype, d, G, s, n, B=2, hkv=2, pad=0.15, dead=0.1):
    hq = G * hkv
    q = torch.from_numpy(rng.standard_normal((B, n, hq, d), dtype=np.float32)).to(dtype)
    k = torch.from_numpy(rng.standard_normal((B, n, hkv, d), dtype=np.float32)).to(dtype)
    v = torch.from_numpy(rng.standard_normal((B, n, hkv, d), dtype=np.float32)).to(dtype)
    do = torch.from_numpy(rng.standard_normal((B, n, hq, d), dtype=np.float32)).to(dtype)
    idx, w = cases.edges(rng, B, n, hkv, s, pad_frac=pad, dead_frac=dead)
    return q, k, v, do, idx, w


@pytest.mark.parametrize("dtype,d,G,s,n", SEA_SHAPES,
                         ids=[f"{str(c[0])[6:]}-d{c[1]}-G{c[2]}-s{c[3]}-n{c[4]}" for c in SEA_SHAPES])
def test_sea_forward_backward_shapes(dtype, d, G, s, n):
    """Each shape twice: the backward recomputing the softmax, and taking the
    forward's p / w statistics (which must also match the oracle's p)."""
    say(f"case sea dtype={dtype} d={d} G={G} s={s} n={n}")
    rng = np.random.default_rng(d * 1000 + G * 100 + s * 10 + n)
    q, k, v, do, idx, w = _sea_inputs(rng, dtype, d, G, s, n)
    orc = oracle.get()
    X = TOL[dtype]
    ro, rp = orc.sea_forward(q, k, v, idx, w, probs=True)
    rdq, rdk, rdv, rdw = orc.sea_backward(q, k, v, idx, w, do)
    dw_err = {}
    for with_stats in (False, True):
        say(f"  stats={with_stats}")
        st = None
        if with_stats:
            o, st = gm.sea_forward(dev(q), dev(k), dev(v), dev(idx), dev(w), save_stats=True)
        else:
            o = gm.sea_forward(dev(q), dev(k), dev(v), dev(idx), dev(w))
        dq, dk, dv, dw = gm.sea_backward(dev(q), dev(k), dev(v), dev(idx), dev(w), dev(do),
                                         stats=st)
        torch.cuda.synchronize()
        assert_close("o", host(o), ro, X)
        if with_stats:
            live = np.repeat(w > 0, G, axis=2)
            hs = host(gm.stats_as_query_heads(st, G))
            assert (hs[~live] == 0).all()
            assert_close("p (statistics * w)", hs * np.repeat(w, G, axis=2), rp, 1e-4)
            ei, ew = gm.stats_edge_copy(st)      # the backward's copy of the edge rows
            assert np.array_equal(host(ei), idx) and np.array_equal(host(ew), w)
        assert_close("dq", host(dq), rdq, X)
        assert_close("dk", host(dk), rdk, X)
        assert_close("dv", host(dv), rdv, X)
        dw_err[with_stats] = assert_close("dw", host(dw), rdw, X)[0]
    # the saved statistics must not cost dw accuracy: the backward forms
    # g_t - gbar without cancellation from either source of p
    assert dw_err[True] <= 10 * dw_err[False] + 1e-6, dw_err


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_sea_single_live_slot_tiny_weights(dtype):
    """Rows with one live slot of tiny weight (as deep referral chains leave):
    p = 1 there, so g - gbar = 0 and dq, dw and that row's dk contribution
    are exactly 0, however large p / w is, with the softmax recomputed or
    taken from the forward's statistics."""
    say(f"case single live slot, tiny weights, {dtype}")
    rng = np.random.default_rng(21)
    q, k, v, do, idx, w = _sea_inputs(rng, dtype, 128, 2, 4, 300, pad=0.0, dead=0.0)
    w[..., 1:] = 0.0
    idx[..., 1:] = 0
    w[..., 0] = (10.0 ** rng.uniform(-9, -3, size=w[..., 0].shape)).astype(np.float32)
    _, st = gm.sea_forward(dev(q), dev(k), dev(v), dev(idx), dev(w), save_stats=True)
    for stats in (None, st):
        dq, dk, dv, dw = gm.sea_backward(dev(q), dev(k), dev(v), dev(idx), dev(w), dev(do),
                                         stats=stats)
        torch.cuda.synchronize()
        say(f"  stats={stats is not None}: max |dw| {np.abs(host(dw)).max():.3e}")
        assert (host(dw) == 0).all() and (host(dq) == 0).all() and (host(dk) == 0).all()
    rdv = oracle.get().sea_backward(q, k, v, idx, w, do)[2]
    assert_close("dv", host(dv), rdv, TOL[dtype])


def test_sea_scale_argument_and_all_padding_rows():
    """A caller-chosen scale, rows whose slots are all padding (o = 0 and no
    gradient) and token 0 (every edge points at itself)."""
    rng = np.random.default_rng(5)
    q, k, v, do, idx, w = _sea_inputs(rng, torch.float32, 64, 2, 4, 30, pad=0.0, dead=0.0)
    idx[:, 7] = 0; w[:, 7] = 0.0
    idx[0, 11, 1] = 0; w[0, 11, 1] = 0.0
    o = gm.sea_forward(dev(q), dev(k), dev(v), dev(idx), dev(w), scale=0.3)
    grads = gm.sea_backward(dev(q), dev(k), dev(v), dev(idx), dev(w), dev(do), scale=0.3)
    orc = oracle.get()
    assert_close("o", host(o), orc.sea_forward(q, k, v, idx, w, scale=0.3), 1e-5)
    for name, g, r in zip(("dq", "dk", "dv", "dw"), grads,
                          orc.sea_backward(q, k, v, idx, w, do, scale=0.3)):
        assert_close(name, host(g), r, 1e-5)
    assert (host(o)[:, 7] == 0).all() and (host(grads[0])[:, 7] == 0).all()


SER_SHAPES = [
    # s1, s2, s3, n, ties
    (4, 4, 4, 70, False),
    (2, 4, 4, 70, True),      # the narrower budget: top-2 of 16
    (4, 4, 4, 70, True),      # exact ties everywhere: lower index first
    (3, 3, 5, 45, False),     # 15 candidates in a 16-lane team
    (8, 8, 8, 33, True),      # a full wave of 64 candidates
    (6, 1, 3, 40, False),     # more slots than candidates: padding
    (1, 2, 2, 129, False),    # 32 units per workgroup, ragged tail
    (5, 2, 3, 50, True),
    (64, 8, 8, 12, False),    # the widest output
]


@pytest.mark.parametrize("s1,s2,s3,n,ties", SER_SHAPES,
                         ids=[f"s{c[0]}-{c[1]}x{c[2]}-n{c[3]}{'-ties' if c[4] else ''}" for c in SER_SHAPES])
def test_ser_forward_backward_shapes(s1, s2, s3, n, ties):
    say(f"case ser s1={s1} s2={s2} s3={s3} n={n} ties={ties}")
    rng = np.random.default_rng(s1 * 1000 + s2 * 100 + s3 * 10 + n)
    B, hkv = 2, 3
    idx1, w1 = cases.edges(rng, B, n, hkv, s2, pad_frac=0.1, ties=ties, dead_frac=0.05)
    idx2, w2 = cases.edges(rng, B, n, hkv, s3, pad_frac=0.1, ties=ties, dead_frac=0.05)
    io, wo = gm.ser_forward(dev(idx1), dev(w1), dev(idx2), dev(w2), s1)
    orc = oracle.get()
    rio, rwo = orc.ser_forward(idx1, w1, idx2, w2, s1)
    assert_ser_match(host(io), host(wo), rio, rwo)
    np.testing.assert_array_equal(host(wo), rwo)
    dwo = rng.standard_normal(rio.shape).astype(np.float32)
    d1, d2 = gm.ser_backward(dev(idx1), dev(w1), dev(idx2), dev(w2), io, wo, dev(dwo))
    r1, r2 = orc.ser_backward(idx1, w1, idx2, w2, rio, rwo, dwo)
    assert_close("dw1", host(d1), r1, 1e-5)
    assert_close("dw2", host(d2), r2, 1e-5)
    if s2 == s3:
        idx2, w2 = idx1, w1
        io, wo = gm.ser_forward(dev(idx1), dev(w1), dev(idx1), dev(w1), s1)
        rio, rwo = orc.ser_forward(idx1, w1, idx1, w1, s1)
        assert_ser_match(host(io), host(wo), rio, rwo)
        da, _ = gm.ser_backward(dev(idx1), dev(w1), dev(idx1), dev(w1), io, wo, dev(dwo),
                                aliased=True)
        ra, _ = orc.ser_backward(idx1, w1, idx1, w1, rio, rwo, dwo, aliased=True)
        assert_close("dw (aliased legs)", host(da), ra, 1e-5)


@pytest.mark.parametrize("n,s1", [(1024, 4), (1025, 4), (2500, 4), (3000, 2), (4096, 4),
                                  (4097, 4), (9000, 4), (13000, 2)])
def test_ser_backward_source_chunks(n, s1):
    """s2 = s3 = 4 backward across the 1024-source chunk boundaries of the
    partial-sum path (n <= 4096; whole-pair LDS accumulators) and past its
    limit (the fp64-atomic path); s1 = 4 and 2, separate and aliased legs."""
    say(f"case ser backward chunks n={n} s1={s1}")
    rng = np.random.default_rng(4000 + n)
    B, hkv = 1, 2
    idx1, w1 = cases.edges(rng, B, n, hkv, 4, pad_frac=0.05, dead_frac=0.05)
    idx2, w2 = cases.edges(rng, B, n, hkv, 4, pad_frac=0.05, dead_frac=0.05)
    orc = oracle.get()
    for legs in ("separate", "aliased"):
        if legs == "aliased":
            idx2, w2 = idx1, w1
        io, wo = gm.ser_forward(dev(idx1), dev(w1), dev(idx2), dev(w2), s1)
        rio, rwo = orc.ser_forward(idx1, w1, idx2, w2, s1)
        assert_ser_match(host(io), host(wo), rio, rwo)
        dwo = rng.standard_normal(rio.shape).astype(np.float32)
        d1, d2 = gm.ser_backward(dev(idx1), dev(w1), dev(idx2), dev(w2), io, wo, dev(dwo),
                                 aliased=legs == "aliased")
        r1, r2 = orc.ser_backward(idx1, w1, idx2, w2, rio, rwo, dwo, aliased=legs == "aliased")
        assert_close(f"dw1 ({legs})", host(d1), r1, 1e-5)
        if legs == "separate":
            assert_close("dw2", host(d2), r2, 1e-5)


PARTITIONED = [(4097, 4, torch.bfloat16, 128), (9000, 4, torch.bfloat16, 128),
               (12289, 3, torch.bfloat16, 128),
               (5000, 4, torch.bfloat16, 256),    # 512-byte rows
               (4600, 3, torch.bfloat16, 64),     # 128-byte rows
               (4500, 2, torch.float32, 128)]     # 512-byte fp32 rows


@pytest.mark.parametrize("n,s,dtype,d", PARTITIONED,
                         ids=[f"n{c[0]}-s{c[1]}-{str(c[2])[6:]}-d{c[3]}" for c in PARTITIONED])
def test_sea_backward_partitioned_index(n, s, dtype, d):
    """n > 4096: the reverse edge index is built by target bucket (512 rows)
    and source chunk (4096 tokens); ragged last bucket and chunk, s = 4 (16-byte
    edge rows) and s = 3; every output compared, with the softmax recomputed
    and with the forward's statistics."""
    say(f"case sea backward partitioned index n={n} s={s} dtype={dtype} d={d}")
    rng = np.random.default_rng(5000 + n + s)
    q, k, v, do, idx, w = _sea_inputs(rng, dtype, d, 2, s, n, B=1, hkv=2)
    rdq, rdk, rdv, rdw = oracle.get().sea_backward(q, k, v, idx, w, do)
    X = TOL[dtype]
    _, st = gm.sea_forward(dev(q), dev(k), dev(v), dev(idx), dev(w), save_stats=True)
    for stats in (None, st):
        say(f"  stats={stats is not None}")
        dq, dk, dv, dw = gm.sea_backward(dev(q), dev(k), dev(v), dev(idx), dev(w), dev(do),
                                         stats=stats)
        assert_close("dq", host(dq), rdq, X)
        assert_close("dk", host(dk), rdk, X)
        assert_close("dv", host(dv), rdv, X)
        assert_close("dw", host(dw), rdw, X)


def test_sea_backward_beyond_partitioned_index():
    """n = 2^20 + 37 tokens (one pair, fp32, d = 64: 256-byte rows): beyond
    the partitioned index's 2^20 rows the row kernels count in-degrees in
    the source pass, scan them over the whole tensor, and reduce every K/V
    row with the persistent target kernel; every output compared with the
    oracle, with and without the forward's statistics."""
    n, s, d = (1 << 20) + 37, 4, 64
    say(f"case sea backward beyond the partitioned index n={n} s={s} fp32 d={d}")
    rng = np.random.default_rng(1 << 20)
    q, k, v, do, idx, w = _sea_inputs(rng, torch.float32, d, 1, s, n, B=1, hkv=1)
    rdq, rdk, rdv, rdw = oracle.get().sea_backward(q, k, v, idx, w, do)
    X = TOL[torch.float32]
    dq_, dk_, dv_, do_ = dev(q), dev(k), dev(v), dev(do)
    di, dw_ = dev(idx), dev(w)
    _, st = gm.sea_forward(dq_, dk_, dv_, di, dw_, save_stats=True)
    for stats in (None, st):
        say(f"  stats={stats is not None}")
        dq, dk, dv, dw = gm.sea_backward(dq_, dk_, dv_, di, dw_, do_, stats=stats)
        assert_close("dq", host(dq), rdq, X)
        assert_close("dk", host(dk), rdk, X)
        assert_close("dv", host(dv), rdv, X)
        assert_close("dw", host(dw), rdw, X)


def _unaligned(x: np.ndarray) -> torch.Tensor:
    """x on the GPU, starting 4 bytes past a 16-byte boundary (contiguous)."""
    flat = torch.empty(x.size + 1, dtype=torch.from_numpy(x[:0].copy()).dtype, device="cuda")
    t = flat[1:].view(x.shape)
    t.copy_(torch.from_numpy(np.ascontiguousarray(x)))
    assert t.data_ptr() % 16 != 0
    return t


def test_unaligned_edge_rows_take_the_scalar_loads():
    """s = 4 edges whose rows are not 16-byte aligned: the forward, source and
    index kernels load slots one by one, SER forward and backward take their
    general lane-per-unit / reverse-index paths; results as for the oracle."""
    say("case unaligned s=4 edges")
    rng = np.random.default_rng(77)
    dtype, d, G, s, n, B, hkv = torch.bfloat16, 128, 2, 4, 300, 2, 2
    q, k, v, do, idx, w = _sea_inputs(rng, dtype, d, G, s, n, B=B, hkv=hkv)
    orc = oracle.get()
    ui, uw = _unaligned(idx), _unaligned(w)
    io, wo = gm.ser_forward(ui, uw, ui, uw, s)
    rio, rwo = orc.ser_forward(idx, w, idx, w, s)
    assert_ser_match(host(io), host(wo), rio, rwo)
    np.testing.assert_array_equal(host(wo), rwo)
    ai, aw = _unaligned(rio), _unaligned(rwo)
    o = gm.sea_forward(dev(q), dev(k), dev(v), ai, aw)
    dq, dk, dv, dw = gm.sea_backward(dev(q), dev(k), dev(v), ai, aw, dev(do))
    X = TOL[dtype]
    assert_close("o", host(o), orc.sea_forward(q, k, v, rio, rwo), X)
    rdq, rdk, rdv, rdw = orc.sea_backward(q, k, v, rio, rwo, do)
    assert_close("dq", host(dq), rdq, X)
    assert_close("dk", host(dk), rdk, X)
    assert_close("dv", host(dv), rdv, X)
    assert_close("dw", host(dw), rdw, X)
    dwo = rng.standard_normal(rio.shape).astype(np.float32)
    da, _ = gm.ser_backward(ui, uw, ui, uw, ai, aw, _unaligned(dwo), aliased=True)
    ra, _ = orc.ser_backward(idx, w, idx, w, rio, rwo, dwo, aliased=True)
    assert_close("dw (aliased legs)", host(da), ra, 1e-5)


def test_single_token_and_empty_inputs():
    """n = 1 (every edge is the padding token itself) and zero-size calls,
    which launch nothing and return success."""
    rng = np.random.default_rng(9)
    q, k, v, do, idx, w = _sea_inputs(rng, torch.bfloat16, 128, 2, 4, 1, pad=0.0, dead=0.0)
    assert (idx == 0).all()
    o = gm.sea_forward(dev(q), dev(k), dev(v), dev(idx), dev(w))
    orc = oracle.get()
    assert_close("o (n=1)", host(o), orc.sea_forward(q, k, v, idx, w), 2e-2)
    io, wo = gm.ser_forward(dev(idx), dev(w), dev(idx), dev(w), 4)
    rio, rwo = orc.ser_forward(idx, w, idx, w, 4)
    assert_ser_match(host(io), host(wo), rio, rwo)
    for B, n in ((0, 16), (2, 0)):
        e_i = torch.zeros((B, n, 2, 4), dtype=torch.int32, device="cuda")
        e_w = torch.zeros((B, n, 2, 4), dtype=torch.float32, device="cuda")
        qq = torch.zeros((B, n, 4, 128), dtype=torch.bfloat16, device="cuda")
        kk = torch.zeros((B, n, 2, 128), dtype=torch.bfloat16, device="cuda")
        gm.ser_forward(e_i, e_w, e_i, e_w, 4)
        gm.sea_forward(qq, kk, kk, e_i, e_w)
        gm.sea_backward(qq, kk, kk, e_i, e_w, qq)
        gm.ser_backward(e_i, e_w, e_i, e_w, e_i, e_w, e_w, aliased=True)
    torch.cuda.synchronize()


def test_forward_calls_are_bitwise_deterministic():
    rng = np.random.default_rng(10)
    q, k, v, do, idx, w = _sea_inputs(rng, torch.bfloat16, 128, 2, 4, 500, B=4, pad=0, dead=0)
    args = [dev(x) for x in (q, k, v, idx, w)]
    a = gm.ser_forward(args[3], args[4], args[3], args[4], 4)
    b = gm.ser_forward(args[3], args[4], args[3], args[4], 4)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    o1 = gm.sea_forward(*args[:3], *a)
    o2 = gm.sea_forward(*args[:3], *a)
    assert torch.equal(o1, o2)


def test_check_edges_counts():
    rng = np.random.default_rng(11)
    idx, w = cases.edges(rng, 2, 100, 3, 4, pad_frac=0.2)
    bad, live = gm.check_edges(dev(idx), dev(w))
    assert bad == 0 and live == int((w > 0).sum())
    idx[1, 5, 2, 1] = 6          # index beyond its own token
    w[0, 9, 0, 3] = -1.0         # negative weight
    w[0, 10, 0, 0] = np.inf
    bad, _ = gm.check_edges(dev(idx), dev(w))
    assert bad == 3


def test_errors_are_reported_before_any_launch():
    idx = torch.zeros((1, 8, 2, 4), dtype=torch.int32, device="cuda")
    w = torch.zeros((1, 8, 2, 4), dtype=torch.float32, device="cuda")
    q = torch.zeros((1, 8, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gm.GMError, match="ALIAS"):
        gm.gm_ser_forward(idx, w, idx, w, idx, w)
    with pytest.raises(gm.GMError, match="UNSUPPORTED"):
        gm.ser_forward(torch.zeros((1, 8, 2, 9), dtype=torch.int32, device="cuda"),
                       torch.zeros((1, 8, 2, 9), dtype=torch.float32, device="cuda"),
                       torch.zeros((1, 8, 2, 9), dtype=torch.int32, device="cuda"),
                       torch.zeros((1, 8, 2, 9), dtype=torch.float32, device="cuda"), 4)
    flat = torch.zeros(q.numel() + 8, dtype=torch.bfloat16, device="cuda")
    misaligned = flat[1:1 + q.numel()].view(q.shape)      # 2 bytes past a 16-byte boundary
    assert misaligned.is_contiguous() and misaligned.data_ptr() % 16 == 2
    with pytest.raises(gm.GMError, match="ALIGN"):
        gm.gm_sea_forward(misaligned, k, k, idx, w, q)
    with pytest.raises(gm.GMError, match="UNSUPPORTED"):     # 5 query heads on 2 KV heads
        gm.sea_forward(torch.zeros((1, 8, 5, 128), dtype=torch.bfloat16, device="cuda"),
                       k, k, idx, w)
    torch.cuda.synchronize()


def test_sea_backward_long_incoming_segments():
    """Every edge of every token points at token 0 or 1, so two K/V rows per
    pair receive thousands of incoming edges (as deep referral chains do)."""
    rng = np.random.default_rng(12)
    q, k, v, do, idx, w = _sea_inputs(rng, torch.bfloat16, 128, 2, 4, 700, pad=0.0, dead=0.0)
    idx = np.minimum(rng.integers(0, 2, size=idx.shape), np.arange(700).reshape(1, 700, 1, 1))
    idx = idx.astype(np.int32)
    grads = gm.sea_backward(dev(q), dev(k), dev(v), dev(idx), dev(w), dev(do))
    torch.cuda.synchronize()
    ref = oracle.get().sea_backward(q, k, v, idx, w, do)
    for name, g, r in zip(("dq", "dk", "dv", "dw"), grads, ref):
        assert_close(name, host(g), r, 2e-2)


DETERMINISM = [("metric", None), ("long64k", None), ("general-G3", (torch.bfloat16, 128, 3, 4, 700)),
               ("general-f32-s9", (torch.float32, 32, 4, 9, 500)),
               ("partitioned", (torch.bfloat16, 128, 2, 4, 9000))]


@pytest.mark.parametrize("case,shape", DETERMINISM, ids=[c[0] for c in DETERMINISM])
def test_sea_backward_bitwise_deterministic(case, shape):
    """Two backward calls on the same inputs give bitwise equal dq, dk, dv and
    dw: every dk/dv row is summed over its incoming edges in ascending edge
    id order (the reverse index fixes that order), whatever order the index
    kernels' atomics placed them in.  Full size for the measured pass and the
    long sequence; a forward run in between changes the caches' state."""
    say(f"case backward determinism {case}")
    if shape is None:
        p = synth.PRESETS[case]
        inp = Inputs(p)
        idx, w = dev(inp.idx), dev(inp.w)
        ia, wa = gm.ser_forward(idx, w, idx, w, p.s1)
        q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout)
    else:
        dtype, d, G, s, n = shape
        rng = np.random.default_rng(31)
        qn, kn, vn, don, idxn, wn = _sea_inputs(rng, dtype, d, G, s, n, B=2, hkv=2)
        q, k, v, do, ia, wa = (dev(x) for x in (qn, kn, vn, don, idxn, wn))
    o, st = gm.sea_forward(q, k, v, ia, wa, save_stats=True)
    first = gm.sea_backward(q, k, v, ia, wa, do, stats=st)
    gm.sea_forward(q, k, v, ia, wa)
    second = gm.sea_backward(q, k, v, ia, wa, do, stats=st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dw"), first, second):
        assert torch.equal(a, b), f"{name} differs between two runs"
    say("  dq, dk, dv, dw bitwise equal")


def test_sea_backward_bucketed_index_concentrated_targets():
    """n = 9000 (the bucketed index) with every edge pointing at token 0 or 1:
    the first bucket holds more edges than LDS can stage, so its rows are
    put in order in global memory, and both rows exceed what one wavefront
    sorts in registers.  Outputs against the oracle; two calls bitwise equal."""
    say("case bucketed index, all edges on tokens 0 and 1")
    rng = np.random.default_rng(13)
    n = 9000
    q, k, v, do, idx, w = _sea_inputs(rng, torch.bfloat16, 128, 2, 4, n, B=1, hkv=2,
                                      pad=0.0, dead=0.0)
    idx = np.minimum(rng.integers(0, 2, size=idx.shape), np.arange(n).reshape(1, n, 1, 1))
    idx = idx.astype(np.int32)
    args = [dev(x) for x in (q, k, v, idx, w, do)]
    first = gm.sea_backward(*args)
    second = gm.sea_backward(*args)
    torch.cuda.synchronize()
    ref = oracle.get().sea_backward(q, k, v, idx, w, do)
    for name, g, g2, r in zip(("dq", "dk", "dv", "dw"), first, second, ref):
        assert torch.equal(g, g2), f"{name} differs between two runs"
        assert_close(name, host(g), r, 2e-2)


def _host_path_map(idx1, w1, idx2, w2, io, wo):
    """The path map written out from its definition (numpy, on the oracle's
    A'): nibble k = 4a + c of unit (b, i, h) is the slot t of A' whose index
    is path (a, c)'s target, when both leg weights are positive and w'_t > 0,
    else 15 (also for k beyond the s2 x s3 paths)."""
    B, n, hkv, s2 = idx1.shape
    s3, s1 = idx2.shape[-1], io.shape[-1]
    bb = np.arange(B).reshape(B, 1, 1)
    hh = np.arange(hkv).reshape(1, 1, hkv)
    mp = np.full((B, n, hkv), np.uint64(0xFFFFFFFFFFFFFFFF), dtype=np.uint64)   # 15: no path
    for a in range(s2):
        j = idx1[..., a]
        for c in range(s3):
            m = idx2[bb, j, hh, c]
            ok = (w1[..., a] > 0) & (w2[bb, j, hh, c] > 0)
            sl = np.full((B, n, hkv), 15, dtype=np.uint64)
            for t in range(s1):
                sl = np.where(ok & (wo[..., t] > 0) & (io[..., t] == m), np.uint64(t), sl)
            sh = np.uint64(4 * (4 * a + c))
            mp = (mp & ~(np.uint64(15) << sh)) | (sl << sh)
    return mp


@pytest.mark.parametrize("s1,s2,s3,n,ties", [(4, 4, 4, 2500, False), (2, 4, 4, 1100, True),
                                             (3, 2, 3, 300, False), (4, 4, 4, 70, True),
                                             (4, 4, 4, 5000, False)])
def test_ser_path_map(s1, s2, s3, n, ties):
    """The SER forward's path map equals its definition (computed on the
    host from the oracle's A'), and the SER backward gives the same
    gradients with and without it, for separate and aliased legs: bitwise
    on the source-chunk path (n <= 4096), within rounding on the fp64-atomic
    path beyond (its atomics add in an order that varies)."""
    say(f"case SER path map s={s1}/{s2}/{s3} n={n} ties={ties}")
    rng = np.random.default_rng(6000 + n)
    B, hkv = 2, 3
    idx1, w1 = cases.edges(rng, B, n, hkv, s2, pad_frac=0.05, ties=ties, dead_frac=0.05)
    idx2, w2 = cases.edges(rng, B, n, hkv, s3, pad_frac=0.05, ties=ties, dead_frac=0.05)
    orc = oracle.get()
    for legs in ("separate", "aliased"):
        if legs == "aliased":
            if s2 != s3:
                continue
            idx2, w2 = idx1, w1
        io, wo, pm = gm.ser_forward(dev(idx1), dev(w1), dev(idx2), dev(w2), s1, save_paths=True)
        rio, rwo = orc.ser_forward(idx1, w1, idx2, w2, s1)
        assert_ser_match(host(io), host(wo), rio, rwo)
        ref = _host_path_map(idx1, w1, idx2, w2, rio, rwo)
        got = pm.cpu().numpy().view(np.uint64)
        assert np.array_equal(got, ref), f"path map differs ({legs} legs)"
        dwo = dev(rng.standard_normal(rio.shape).astype(np.float32))
        al = legs == "aliased"
        with_map = gm.ser_backward(dev(idx1), dev(w1), dev(idx2), dev(w2), io, wo, dwo,
                                   aliased=al, paths=pm)
        without = gm.ser_backward(dev(idx1), dev(w1), dev(idx2), dev(w2), io, wo, dwo,
                                  aliased=al)
        torch.cuda.synchronize()
        for a_, b_ in zip(with_map, without):
            if n <= 4096:
                assert torch.equal(a_, b_), f"SER backward with the path map differs ({legs} legs)"
            else:
                assert torch.allclose(a_, b_, rtol=1e-6, atol=1e-7), f"{legs} legs"
        r1, r2 = orc.ser_backward(idx1, w1, idx2, w2, rio, rwo, host(dwo), aliased=al)
        assert_close(f"dw1 ({legs}, path map)", host(with_map[0]), r1, 1e-5)
        if not al:
            assert_close("dw2 (path map)", host(with_map[1]), r2, 1e-5)
