"""GPU parity of the decode step (gm_decode_step) against the oracle.

The oracle has no decode function; it runs the training-pass definition on
whole sequences whose row t_b (one chosen position per sequence) holds the
decoded token's leg-1 row and query, and the decode step must reproduce that
row: SER indices and weights bit-exact, o within the SEA bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cases
import oracle
import sparse_dynamic_routing_amd as gm
from gpu_util import TOL, assert_close, assert_ser_match, dev, host, say

pytestmark = pytest.mark.gpu

DECODE_CASES = [
    # dtype, d, G, s1, s2, s3, B, T
    (torch.bfloat16, 128, 2, 4, 4, 4, 4, 300),    # the measured layer's budget
    (torch.bfloat16, 128, 2, 2, 4, 4, 3, 200),    # top-2 of 16
    (torch.float32, 64, 4, 3, 3, 5, 2, 77),       # 15 candidates, fp64 arithmetic
    (torch.bfloat16, 256, 1, 8, 8, 8, 2, 150),    # a full wave of candidates
    (torch.float32, 16, 16, 64, 8, 8, 2, 40),     # the widest output: padding
    (torch.bfloat16, 32, 8, 1, 2, 2, 5, 1),       # a one-token cache
    # bf16, d = 128, <= 16 candidates: the kernel that loads every
    # candidate's K/V rows while SER ranks them
    (torch.bfloat16, 128, 1, 3, 3, 5, 2, 90),     # 15 candidates, one query head
    (torch.bfloat16, 128, 4, 8, 2, 8, 3, 120),    # 16 candidates, more slots than kept ones
    (torch.bfloat16, 128, 2, 1, 1, 1, 2, 10),     # a single candidate
]


@pytest.mark.parametrize("dtype,d,G,s1,s2,s3,B,T", DECODE_CASES,
                         ids=[f"{str(c[0])[6:]}-d{c[1]}-G{c[2]}-s{c[3]}-{c[4]}x{c[5]}-T{c[7]}"
                              for c in DECODE_CASES])
def test_decode_step_matches_training_definition(dtype, d, G, s1, s2, s3, B, T):
    say(f"case decode dtype={dtype} d={d} G={G} s=({s1},{s2},{s3}) B={B} T={T}")
    rng = np.random.default_rng(d * 100 + G * 10 + s1 + T)
    hkv = 2
    hq = G * hkv
    idx1, w1 = cases.edges(rng, B, T, hkv, s2, pad_frac=0.1, dead_frac=0.05)
    idx2, w2 = cases.edges(rng, B, T, hkv, s3, pad_frac=0.1, dead_frac=0.05,
                           ties=bool(s1 % 2))
    q = torch.from_numpy(rng.standard_normal((B, T, hq, d), dtype=np.float32)).to(dtype)
    k = torch.from_numpy(rng.standard_normal((B, T, hkv, d), dtype=np.float32)).to(dtype)
    v = torch.from_numpy(rng.standard_normal((B, T, hkv, d), dtype=np.float32)).to(dtype)
    tpos = rng.integers(0, T, size=B)
    tpos[0] = T - 1
    bi = np.arange(B)
    # the decoded tokens: their leg-1 rows and queries
    d_idx1 = np.ascontiguousarray(idx1[bi, tpos])
    d_w1 = np.ascontiguousarray(w1[bi, tpos])
    d_q = q[torch.from_numpy(bi), torch.from_numpy(tpos)].contiguous()
    io, wo, o = gm.decode_step(dev(d_idx1), dev(d_w1), dev(idx2), dev(w2), dev(d_q), dev(k),
                               dev(v), s1)
    torch.cuda.synchronize()
    orc = oracle.get()
    rio, rwo = orc.ser_forward(idx1, w1, idx2, w2, s1)
    ro = orc.sea_forward(q, k, v, rio, rwo)
    assert_ser_match(host(io)[:, None], host(wo)[:, None],
                     rio[bi, tpos][:, None], rwo[bi, tpos][:, None])
    np.testing.assert_array_equal(host(wo), rwo[bi, tpos])
    assert_close("o", host(o), ro[bi, tpos], TOL[dtype])


def test_decode_step_matches_the_training_kernels():
    """Leg 1 = the cache's own row at the last position (A' = Sp(A A)): the
    decode step gives the training kernels' last row (SER bitwise, o to the
    bf16 bar: the two kernels round differently)."""
    rng = np.random.default_rng(77)
    B, T, hkv, G, d, s = 3, 513, 8, 2, 128, 4
    idx, w = cases.edges(rng, B, T, hkv, s, pad_frac=0.05)
    q = dev(torch.from_numpy(rng.standard_normal((B, T, hkv * G, d), dtype=np.float32))
            .to(torch.bfloat16))
    k = dev(torch.from_numpy(rng.standard_normal((B, T, hkv, d), dtype=np.float32))
            .to(torch.bfloat16))
    v = dev(torch.from_numpy(rng.standard_normal((B, T, hkv, d), dtype=np.float32))
            .to(torch.bfloat16))
    di, dw = dev(idx), dev(w)
    ia, wa = gm.ser_forward(di, dw, di, dw, s)
    o = gm.sea_forward(q, k, v, ia, wa)
    io, wo, od = gm.decode_step(di[:, -1].contiguous(), dw[:, -1].contiguous(), di, dw,
                                q[:, -1].contiguous(), k, v, s)
    torch.cuda.synchronize()
    assert torch.equal(io, ia[:, -1]) and torch.equal(wo, wa[:, -1])
    assert_close("o", host(od), host(o[:, -1]), TOL[torch.bfloat16])
