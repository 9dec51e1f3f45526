"""The C-ABI library without a GPU: it loads, exports every call that
include/gm.h declares, and rejects bad arguments on the host before any
launch (these calls never reach HIP, so they run on a CPU-only machine)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import sparse_dynamic_routing_amd as gm
from sparse_dynamic_routing_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gm.h")

OK, NULL, SHAPE, UNSUP, WS, HIP, ALIGN, ALIAS = range(8)


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gm_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return gm.load()


def test_library_exports_every_declared_call(lib):
    names = declared()
    assert names, "no declarations found in gm.h"
    assert set(names) == set(binding.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.gm_abi_version() == 8


def test_status_strings(lib):
    for code in range(9):
        assert lib.gm_status_string(code)
    assert b"unknown" in lib.gm_status_string(99)


P = ctypes.c_void_p


def fake(addr):
    """A non-NULL pointer value that is never dereferenced (the host checks
    reject the call before any launch)."""
    return P(addr)


def test_ser_forward_argument_checks(lib):
    a = fake(0x10000)
    f = lib.gm_ser_forward
    assert f(-1, 4, 1, a, a, 2, a, a, 2, a, a, 2, None, None) == SHAPE
    assert f(1, 4, 1, a, a, 2, a, a, 2, a, a, 0, None, None) == UNSUP       # s1 = 0
    assert f(1, 4, 1, a, a, 9, a, a, 8, a, a, 4, None, None) == UNSUP       # 72 candidates
    assert f(1, 4, 1, a, a, 2, a, a, 2, a, a, 65, None, None) == UNSUP
    assert f(1, 4, 1, None, a, 2, a, a, 2, a, a, 2, None, None) == NULL
    assert f(1, 4, 1, fake(0x10002), a, 2, a, a, 2, fake(0x20000), fake(0x30000), 2,
             None, None) == ALIGN
    assert f(1, 4, 1, a, fake(0x40000), 2, a, fake(0x40000), 2, a, fake(0x50000), 2,
             None, None) == ALIAS                                           # idx_out on idx1
    assert f(0, 4, 1, None, None, 2, None, None, 2, None, None, 2, None, None) == OK  # empty
    assert f(70000, 70000, 1, a, a, 2, a, a, 2, a, a, 2, None, None) == SHAPE  # > 2^31 units
    far = [fake(k << 32) for k in range(1, 8)]
    assert f(1, 4, 1, *far[:2], 4, *far[2:4], 8, *far[4:6], 4, far[6], None) == UNSUP  # paths: s3 > 4
    assert f(1, 4, 1, *far[:2], 4, *far[2:4], 4, *far[4:6], 4, fake((8 << 32) + 4),
             None) == ALIGN                                           # paths 8-byte aligned
    assert f(1, 4, 1, *far[:2], 4, *far[2:4], 4, *far[4:6], 4, far[0], None) == ALIAS


def test_ser_forward_chain2_argument_checks(lib):
    f = lib.gm_ser_forward_chain2
    i, w, io, wo = (fake(k << 32) for k in range(1, 5))
    im, wm = fake(5 << 32), fake(6 << 32)
    assert f(-1, 4, 1, i, w, 4, None, None, io, wo, None) == SHAPE
    assert f(1, 4, 1, i, w, 3, None, None, io, wo, None) == UNSUP        # s = 3
    assert f(1, 4, 1, i, w, 8, None, None, io, wo, None) == UNSUP        # s = 8
    assert f(0, 4, 1, None, None, 4, None, None, None, None, None) == OK  # empty
    assert f(1, 4, 1, None, w, 4, None, None, io, wo, None) == NULL
    assert f(1, 4, 1, i, w, 4, im, None, io, wo, None) == NULL           # half of A1
    assert f(1, 4, 1, fake((1 << 32) + 8), w, 4, None, None, io, wo, None) == ALIGN
    assert f(1, 4, 1, i, w, 4, im, fake((6 << 32) + 4), io, wo, None) == ALIGN
    assert f(1, 4, 1, i, w, 4, None, None, i, wo, None) == ALIAS         # A2 on A0
    assert f(1, 4, 1, i, w, 4, io, wm, io, wo, None) == ALIAS            # A1 on A2


def test_sea_argument_checks(lib):
    a, b, c = fake(0x100000), fake(0x200000), fake(0x300000)
    i, w, o = fake(0x400000), fake(0x500000), fake(0x600000)
    f = lib.gm_sea_forward
    args = lambda hq=16, hkv=8, d=128, dt=1, s=4, q=a, oo=o, st=None: (  # noqa: E731
        8, 4096, hq, hkv, d, dt, 0.1, q, b, c, i, w, s, oo, st, None)
    assert f(*args(hq=12)) == UNSUP          # hq % hkv != 0
    assert f(*args(hq=24, q=None)) == NULL   # 3 query heads per KV head: accepted (then NULL)
    assert f(*args(hq=40, q=None)) == NULL   # 5 per KV head
    assert f(*args(d=96)) == UNSUP
    assert f(*args(d=512)) == UNSUP
    assert f(*args(dt=7)) == UNSUP
    assert f(*args(s=0)) == UNSUP
    assert f(*args(s=65)) == UNSUP
    assert f(*args(q=None)) == NULL
    assert f(*args(q=fake(0x100008))) == ALIGN
    assert f(*args(oo=a)) == ALIAS           # o on q
    assert f(*args(st=fake(0x700008))) == ALIGN       # statistics: 16-byte aligned
    assert f(*args(st=b)) == ALIAS           # statistics on k
    g = lib.gm_sea_backward
    need = lib.gm_sea_backward_workspace_bytes(8, 4096, 16, 8, 4)
    assert need >= 8 * 4096 * 8 * 4 * (2 * 8 + 4)      # coefficients and edge list
    ws = fake(0x40000000)
    bargs = [8, 4096, 16, 8, 128, 1, 0.1, a, b, c, i, w, 4, fake(0x700000), None,
             fake(0x800000), fake(0x900000), fake(0xA00000), fake(0xB00000), ws, need, None]
    bad = list(bargs); bad[16] = None
    assert g(*bad) == NULL
    bad = list(bargs); bad[16] = fake(0x900004)
    assert g(*bad) == ALIGN
    bad = list(bargs); bad[15] = b            # dq on k
    assert g(*bad) == ALIAS
    bad = list(bargs); bad[20] = need - 1
    assert g(*bad) == WS
    bad = list(bargs); bad[19] = fake(0x40000010)
    assert g(*bad) == ALIGN
    bad = list(bargs); bad[14] = fake(0xC00004)   # statistics misaligned
    assert g(*bad) == ALIGN
    bad = list(bargs); bad[14] = fake(0x800000)   # dq on the statistics
    assert g(*bad) == ALIAS


def test_decode_step_argument_checks(lib):
    f = lib.gm_decode_step
    i1, w1, i2, w2 = fake(0x100000), fake(0x200000), fake(0x1000000), fake(0x2000000)
    q, k, v = fake(0x300000), fake(0x10000000), fake(0x20000000)
    io, wo, o = fake(0x400000), fake(0x500000), fake(0x600000)
    args = lambda B=8, T=4096, hq=16, hkv=8, d=128, dt=1, s2=4, s3=4, s1=4, qq=q, oo=o: (  # noqa
        B, T, hq, hkv, d, dt, 0.1, i1, w1, s2, i2, w2, s3, s1, qq, k, v, io, wo, oo, None)
    assert f(*args(hq=12)) == UNSUP
    assert f(*args(d=96)) == UNSUP
    assert f(*args(s2=9, s3=8)) == UNSUP       # 72 candidates
    assert f(*args(s1=65)) == UNSUP
    assert f(*args(T=0)) == SHAPE              # an empty cache with tokens to decode
    assert f(*args(B=0)) == OK                 # nothing to decode
    assert f(*args(qq=None)) == NULL
    assert f(*args(qq=fake(0x300008))) == ALIGN
    assert f(*args(oo=q)) == ALIAS             # o on q


def test_dense_refresh_argument_checks(lib):
    f = lib.gm_dense_refresh
    q, k, ls = fake(0x1000000), fake(0x2000000), fake(0x300000)
    io, wo = fake(0x400000), fake(0x500000)
    args = lambda B=8, n=4096, hq=16, hkv=8, d=128, dt=1, s=4, qq=q, kk=k, l=ls, o=io, sc=0.1: (  # noqa
        B, n, hq, hkv, d, dt, sc, qq, kk, s, 0, l, o, wo, None)
    assert f(*args(sc=0.0)) == UNSUP
    assert f(*args(sc=-0.1)) == UNSUP
    assert f(*args(sc=float("inf"))) == UNSUP
    assert f(*args(dt=0)) == UNSUP             # fp32 scores are not offered
    assert f(*args(d=96)) == UNSUP
    assert f(*args(d=256, hq=32)) == UNSUP     # G = 4 at d = 256: too many query registers
    assert f(*args(s=9)) == UNSUP
    assert f(*args(s=0)) == UNSUP
    assert f(*args(hq=12)) == UNSUP
    assert f(*args(n=-1)) == SHAPE
    assert f(*args(B=0)) == OK                 # nothing to do
    assert f(*args(kk=None)) == NULL
    assert f(*args(l=None)) == NULL
    assert f(*args(qq=fake(0x1000008))) == ALIGN
    assert f(*args(o=fake(0x400002))) == ALIGN
    assert f(*args(o=k)) == ALIAS              # idx_out on k
    assert f(*args(l=fake(0x400000 + 4096))) == ALIAS   # lse on idx_out


def test_leg_mix_argument_checks(lib):
    f, g = lib.gm_leg_mix_forward, lib.gm_leg_mix_backward
    i, w, al = fake(0x100000), fake(0x200000), fake(0x300000)
    io, wo = fake(0x400000), fake(0x500000)
    assert f(8, 4096, 8, i, w, 65, al, 4, io, wo, None) == UNSUP     # K > 64
    assert f(8, 4096, 8, i, w, 16, al, 0, io, wo, None) == UNSUP     # s < 1
    assert f(8, 4096, 8, i, w, 16, None, 4, io, wo, None) == NULL
    assert f(8, 4096, 8, i, w, 16, al, 4, i, wo, None) == ALIAS      # idx_out on idx
    assert f(0, 4096, 8, None, None, 16, None, 4, None, None, None) == OK
    need = lib.gm_leg_mix_backward_workspace_bytes(8, 4096, 8, 16)
    assert need == 8 * 1024 * 16 * 8           # fp64 partial per (head, 256 units) at K = 16
    assert lib.gm_leg_mix_backward_workspace_bytes(8, 4096, 8, 24) == 8 * 512 * 24 * 8   # per 64 tokens
    dl, dw, da, ws = fake(0x600000), fake(0x10000000), fake(0x700000), fake(0x20000000)
    args = [8, 4096, 8, i, w, 16, al, io, wo, 4, dl, dw, da, ws, need, None]
    bad = list(args); bad[14] = need - 1
    assert g(*bad) == WS
    bad = list(args); bad[12] = None
    assert g(*bad) == NULL
    bad = list(args); bad[11] = w                                      # dw on w
    assert g(*bad) == ALIAS


def test_ser_backward_workspace_checks(lib):
    need = lib.gm_ser_backward_workspace_bytes(8, 4096, 8, 4, 4, 1)
    acc = 8 * 4096 * 8 * (4 + 4) * 8                       # fp64 dw1 + dw2 accumulators
    part = 8 * 8 * (1024 + 2048 + 3072 + 4096) * 4 * 8     # fp64 partials of 4 source chunks
    assert need == max(acc, part)
    assert lib.gm_ser_backward_workspace_bytes(8, 4096, 8, 4, 4, 0) == need
    ptrs = [fake(0x1000000 * (k + 1)) for k in range(10)]
    args = [8, 4096, 8, ptrs[0], ptrs[1], 4, ptrs[2], ptrs[3], 4, ptrs[4], ptrs[5], 4,
            ptrs[6], None, ptrs[7], ptrs[7], ptrs[8], need - 8, None]
    assert lib.gm_ser_backward(*args) == WS
    args[17] = need; args[16] = None
    assert lib.gm_ser_backward(*args) == WS
    args[16] = fake(0x9000004)
    assert lib.gm_ser_backward(*args) == ALIGN
    args[16] = ptrs[8]
    args[13] = fake(0xA000004)                 # path map misaligned
    assert lib.gm_ser_backward(*args) == ALIGN
    args[13] = ptrs[9]
    args[5] = 2                                # aliased outputs with s2 != s3
    assert lib.gm_ser_backward(*args) == ALIAS


def test_sea_backward_noalloc_checks(lib):
    """The allocation-free backward validates everything on the host first:
    sizes whose workspace exceeds the fixed scratch are GM_ERR_TOO_LARGE, and
    bad pointers are reported as for gm_sea_backward, before any GPU call."""
    a, b, c = fake(0x100000), fake(0x200000), fake(0x300000)
    i, w = fake(0x400000), fake(0x500000)
    f = lib.gm_sea_backward_noalloc
    f.argtypes = [ctypes.c_int] * 6 + [ctypes.c_float] + [P] * 5 + [ctypes.c_int] + [P] * 7
    TOO_LARGE = 8
    args = lambda B=8, n=4096, dq=fake(0x800000), dk=fake(0x900000): (  # noqa: E731
        B, n, 16, 8, 128, 1, 0.1, a, b, c, i, w, 4, fake(0x700000), None,
        dq, dk, fake(0xA00000), fake(0xB00000), None)
    need = lib.gm_sea_backward_workspace_bytes(8, 4096, 16, 8, 4)
    assert need <= 64 << 20                       # the measured layer fits the scratch
    assert lib.gm_sea_backward_workspace_bytes(32, 4096, 16, 8, 4) > 64 << 20
    far = [fake(k << 36) for k in range(1, 11)]   # regions that cannot overlap
    big = (32, 4096, 16, 8, 128, 1, 0.1, *far[:5], 4, far[5], None, *far[6:10], None)
    assert f(*big) == TOO_LARGE
    assert f(*args(dq=None)) == NULL
    assert f(*args(dk=fake(0x900004))) == ALIGN
    assert f(*args(dq=b)) == ALIAS               # dq on k
    assert f(*args(B=0)) == OK                   # empty: nothing to do
    assert b"GM_NOALLOC_SCRATCH_BYTES" in lib.gm_status_string(TOO_LARGE)


def test_gather_probe_library_checks_arguments():
    """The measurement probe (libgm_probe.so) loads and refuses bad arguments
    on the host, before any launch."""
    path = os.path.join(ROOT, "sparse_dynamic_routing_amd", "libgm_probe.so")
    probe = ctypes.CDLL(path)
    f = probe.gm_probe_gather
    f.argtypes = [P, ctypes.c_longlong, P, ctypes.c_longlong, ctypes.c_int, P, ctypes.c_int, P]
    f.restype = ctypes.c_int
    a = fake(0x10000)
    assert f(None, 16, a, 16, 1, a, 8, None) == 1          # no table
    assert f(a, 16, a, 16, 3, a, 8, None) == 1             # 3 loads in flight: not built
    assert f(a, 16, a, 16, 1, a, 12, None) == 1            # grid not a multiple of 8
    assert f(a, 0, a, 16, 1, a, 8, None) == 1              # empty set
