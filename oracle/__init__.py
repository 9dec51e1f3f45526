"""Python access to the C oracle of the Graph Machine sparse-layer path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  The oracle is
plain single-threaded C in double (``gm_oracle.c``, which cites the passages
it follows); this wrapper only converts arrays and calls it.

``build()`` compiles the C file with gcc into ``liboracle.so`` beside it.  It
runs on import when the library is missing or older than its source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_longlong)


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle (plain gcc, no fast-math, no FMA contraction)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-Wall", "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _fresh(lib: str, src: str) -> bool:
    return os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(src)


class OracleError(RuntimeError):
    pass


class Oracle:
    """Handle on one compiled oracle library (the default one, or a test copy)."""

    def __init__(self, path: str = LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_ser_forward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int,
            _i32p, _f64p, ctypes.c_int, _i32p, _f64p, ctypes.c_int,
            ctypes.c_int, _i32p, _f32p, _f64p]
        lib.oracle_sea_forward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, _f64p, _f64p, _f64p, _i32p, _f64p, ctypes.c_int,
            _f64p, _f64p, _i64p]
        lib.oracle_sea_backward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, _f64p, _f64p, _f64p, _i32p, _f64p, ctypes.c_int,
            _f64p, _f64p, _f64p, _f64p, _f64p]
        lib.oracle_ser_backward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int,
            _i32p, _f64p, ctypes.c_int, _i32p, _f64p, ctypes.c_int,
            _i32p, _f64p, ctypes.c_int, _f64p, _f64p, _f64p]
        lib.oracle_leg_mix_forward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _f64p, ctypes.c_int, _f64p,
            ctypes.c_int, _i32p, _f32p]
        lib.oracle_leg_mix_backward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _f64p, ctypes.c_int, _f64p,
            _i32p, _f64p, ctypes.c_int, _f64p, _f64p, _f64p]
        lib.oracle_dense_refresh.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, _f64p, _f64p, ctypes.c_int, _i32p, _f32p, _f64p]
        for f in ("oracle_ser_forward", "oracle_sea_forward",
                  "oracle_sea_backward", "oracle_ser_backward",
                  "oracle_leg_mix_forward", "oracle_leg_mix_backward", "oracle_dense_refresh"):
            getattr(lib, f).restype = ctypes.c_int
        self.lib = lib

    # -- marshalling ----------------------------------------------------
    @staticmethod
    def _np(x, dtype):
        if hasattr(x, "detach"):              # torch tensor (any dtype, CPU)
            x = x.detach().cpu()
            if str(x.dtype) == "torch.bfloat16":
                x = x.float()
            x = x.numpy()
        return np.ascontiguousarray(x, dtype=dtype)

    @staticmethod
    def _p(a, ptype):
        return a.ctypes.data_as(ptype)

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise OracleError(f"{what}: oracle returned {rc} "
                              f"({'index outside [0, i]' if rc == -1 else 'bad arguments'})")

    # -- the four stages -------------------------------------------------
    def ser_forward(self, idx1, w1, idx2, w2, s1, exact=False):
        """A' = Sparsify_s1(A1 A2).  Returns (idx int32, w float32[, w float64])."""
        idx1 = self._np(idx1, np.int32); w1 = self._np(w1, np.float64)
        idx2 = self._np(idx2, np.int32); w2 = self._np(w2, np.float64)
        B, n, hkv, s2 = idx1.shape
        s3 = idx2.shape[-1]
        assert idx2.shape[:3] == (B, n, hkv) and w1.shape == idx1.shape and w2.shape == idx2.shape
        io = np.empty((B, n, hkv, s1), np.int32)
        wo = np.empty((B, n, hkv, s1), np.float32)
        we = np.empty((B, n, hkv, s1), np.float64) if exact else None
        rc = self.lib.oracle_ser_forward(
            B, n, hkv, self._p(idx1, _i32p), self._p(w1, _f64p), s2,
            self._p(idx2, _i32p), self._p(w2, _f64p), s3, s1,
            self._p(io, _i32p), self._p(wo, _f32p),
            self._p(we, _f64p) if exact else None)
        self._check(rc, "ser_forward")
        return (io, wo, we) if exact else (io, wo)

    def sea_forward(self, q, k, v, idx, w, scale=None, count=False, probs=False):
        """o [B,n,hq,d] float64; with ``probs`` also p [B,n,hq,s] (0 on dead
        slots); with ``count`` also the K/V row count (last)."""
        q = self._np(q, np.float64); k = self._np(k, np.float64); v = self._np(v, np.float64)
        idx = self._np(idx, np.int32); w = self._np(w, np.float64)
        B, n, hq, d = q.shape
        hkv, s = idx.shape[2], idx.shape[3]
        scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
        o = np.empty_like(q)
        p = np.empty((B, n, hq, s), np.float64) if probs else None
        rows = ctypes.c_longlong(0)
        rc = self.lib.oracle_sea_forward(
            B, n, hq, hkv, d, scale, self._p(q, _f64p), self._p(k, _f64p),
            self._p(v, _f64p), self._p(idx, _i32p), self._p(w, _f64p), s,
            self._p(o, _f64p), self._p(p, _f64p) if probs else None, ctypes.byref(rows))
        self._check(rc, "sea_forward")
        out = (o,) + ((p,) if probs else ()) + ((rows.value,) if count else ())
        return out if len(out) > 1 else o

    def sea_backward(self, q, k, v, idx, w, dout, scale=None):
        """(dq, dk, dv, dw) in float64."""
        q = self._np(q, np.float64); k = self._np(k, np.float64); v = self._np(v, np.float64)
        idx = self._np(idx, np.int32); w = self._np(w, np.float64)
        dout = self._np(dout, np.float64)
        B, n, hq, d = q.shape
        hkv, s = idx.shape[2], idx.shape[3]
        scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
        dq = np.empty_like(q); dk = np.empty_like(k); dv = np.empty_like(v)
        dw = np.empty(idx.shape, np.float64)
        rc = self.lib.oracle_sea_backward(
            B, n, hq, hkv, d, scale, self._p(q, _f64p), self._p(k, _f64p),
            self._p(v, _f64p), self._p(idx, _i32p), self._p(w, _f64p), s,
            self._p(dout, _f64p), self._p(dq, _f64p), self._p(dk, _f64p),
            self._p(dv, _f64p), self._p(dw, _f64p))
        self._check(rc, "sea_backward")
        return dq, dk, dv, dw

    def ser_backward(self, idx1, w1, idx2, w2, idx_out, w_out, dw_out, aliased=False):
        """(dw1, dw2) in float64; with ``aliased`` both land in one array
        (returned twice), as when A' = Sparsify(A A)."""
        idx1 = self._np(idx1, np.int32); w1 = self._np(w1, np.float64)
        idx2 = self._np(idx2, np.int32); w2 = self._np(w2, np.float64)
        idx_out = self._np(idx_out, np.int32); w_out = self._np(w_out, np.float64)
        dw_out = self._np(dw_out, np.float64)
        B, n, hkv, s2 = idx1.shape
        s3 = idx2.shape[-1]; s1 = idx_out.shape[-1]
        dw1 = np.empty(idx1.shape, np.float64)
        if aliased:
            assert s2 == s3
            dw2 = dw1
        else:
            dw2 = np.empty(idx2.shape, np.float64)
        rc = self.lib.oracle_ser_backward(
            B, n, hkv, self._p(idx1, _i32p), self._p(w1, _f64p), s2,
            self._p(idx2, _i32p), self._p(w2, _f64p), s3,
            self._p(idx_out, _i32p), self._p(w_out, _f64p), s1,
            self._p(dw_out, _f64p), self._p(dw1, _f64p), self._p(dw2, _f64p))
        self._check(rc, "ser_backward")
        return dw1, dw2

    def leg_mix_forward(self, idx, w, alpha, s):
        """Leg of s slots from K stored edges mixed by alpha [hkv, K].
        Returns (idx int32, w float32)."""
        idx = self._np(idx, np.int32); w = self._np(w, np.float64)
        alpha = self._np(alpha, np.float64)
        B, n, hkv, K = idx.shape
        assert w.shape == idx.shape and alpha.shape == (hkv, K)
        io = np.empty((B, n, hkv, s), np.int32)
        wo = np.empty((B, n, hkv, s), np.float32)
        rc = self.lib.oracle_leg_mix_forward(B, n, hkv, self._p(idx, _i32p), self._p(w, _f64p), K,
                                             self._p(alpha, _f64p), s, self._p(io, _i32p),
                                             self._p(wo, _f32p))
        self._check(rc, "leg_mix_forward")
        return io, wo

    def leg_mix_backward(self, idx, w, alpha, idx_out, w_out, dleg):
        """(dw [B,n,hkv,K], dalpha [hkv,K]) in float64."""
        idx = self._np(idx, np.int32); w = self._np(w, np.float64)
        alpha = self._np(alpha, np.float64)
        idx_out = self._np(idx_out, np.int32); w_out = self._np(w_out, np.float64)
        dleg = self._np(dleg, np.float64)
        B, n, hkv, K = idx.shape
        s = idx_out.shape[-1]
        dw = np.empty(idx.shape, np.float64)
        da = np.empty((hkv, K), np.float64)
        rc = self.lib.oracle_leg_mix_backward(
            B, n, hkv, self._p(idx, _i32p), self._p(w, _f64p), K, self._p(alpha, _f64p),
            self._p(idx_out, _i32p), self._p(w_out, _f64p), s, self._p(dleg, _f64p),
            self._p(dw, _f64p), self._p(da, _f64p))
        self._check(rc, "leg_mix_backward")
        return dw, da


    def dense_refresh(self, q, k, s, scale=None):
        """Refresh edges (idx int32, w float32 [B,n,hkv,s]) and the per-head
        log-sum-exp (float64 [B,n,hq]) of dense causal attention."""
        q = self._np(q, np.float64); k = self._np(k, np.float64)
        B, n, hq, d = q.shape
        hkv = k.shape[2]
        scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
        io = np.empty((B, n, hkv, s), np.int32)
        wo = np.empty((B, n, hkv, s), np.float32)
        lse = np.empty((B, n, hq), np.float64)
        rc = self.lib.oracle_dense_refresh(B, n, hq, hkv, d, scale, self._p(q, _f64p),
                                           self._p(k, _f64p), s, self._p(io, _i32p),
                                           self._p(wo, _f32p), self._p(lse, _f64p))
        self._check(rc, "dense_refresh")
        return io, wo, lse


_default: Oracle | None = None


def get() -> Oracle:
    """The default oracle, compiled first if missing or stale."""
    global _default
    if _default is None:
        if not _fresh(LIB, SRC):
            build()
        _default = Oracle(LIB)
    return _default
