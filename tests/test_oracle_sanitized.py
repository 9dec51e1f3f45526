"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and run on small cases of every function, including
the degenerate ones: a single token, padding and dead slots, one slot,
duplicate targets, a group of three query heads, refresh with more slots
than positions.  Any out-of-bounds access, use of freed memory, signed
overflow or other undefined behaviour aborts the child process.

The child loads the instrumented library through the oracle's own ctypes
wrapper (``oracle.Oracle(path)``), with the ASan runtime preloaded, since
the Python interpreter itself is not instrumented."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gm_oracle.c")

CHILD = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, ROOT)
    sys.path.insert(0, TESTS)
    import cases
    import oracle

    orc = oracle.Oracle(LIB)
    rng = np.random.default_rng(7)
    done = 0
    for (B, n, hkv, G, d, s) in [(1, 1, 1, 1, 16, 1), (2, 9, 2, 3, 16, 2), (1, 33, 3, 2, 32, 4),
                                 (2, 17, 1, 1, 16, 3)]:
        for pad, dead, ties, selfl in [(0.0, 0.0, False, 0.0), (0.3, 0.2, True, 0.5)]:
            idx, w = cases.edges(rng, B, n, hkv, s, pad_frac=pad, ties=ties,
                                 self_loop_frac=selfl, dead_frac=dead)
            io, wo = orc.ser_forward(idx, w, idx, w, s)
            io2, wo2, we2 = orc.ser_forward(idx, w, idx, w, s, exact=True)
            hq = G * hkv
            q = rng.standard_normal((B, n, hq, d))
            k = rng.standard_normal((B, n, hkv, d))
            v = rng.standard_normal((B, n, hkv, d))
            do = rng.standard_normal((B, n, hq, d))
            # rows with no live slot are outside the oracle's domain
            live = (wo > 0).any(-1, keepdims=True)
            wo = np.where(live, wo, np.where(np.arange(s) == 0, 1.0, 0.0)).astype(np.float32)
            io = np.where(live, io, 0).astype(np.int32)
            orc.sea_forward(q, k, v, io, wo, count=True, probs=True)
            dq, dk, dv, dw = orc.sea_backward(q, k, v, io, wo, do)
            orc.ser_backward(idx, w, idx, w, io, wo, dw, aliased=True)
            orc.ser_backward(idx, w, idx, w, io, wo, dw, aliased=False)
            done += 1
        K = 3 * s   # stored edges per unit, mixed into a leg of s slots
        idx, w = cases.edges(rng, B, n, hkv, K, pad_frac=0.2, dead_frac=0.1)
        alpha = rng.standard_normal((hkv, K))
        li, lw = orc.leg_mix_forward(idx, w, alpha, s)
        orc.leg_mix_backward(idx, w, alpha, li, lw, rng.standard_normal(li.shape))
        orc.dense_refresh(rng.standard_normal((B, n, G * hkv, d)),
                          rng.standard_normal((B, n, hkv, d)), min(4, n + 2))
    print("sanitized oracle ok", done)
""")


def _have_gcc_sanitizers() -> bool:
    if not shutil.which("gcc"):
        return False
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    return r.returncode == 0 and os.path.isabs(r.stdout.strip())


@pytest.mark.skipif(not _have_gcc_sanitizers(), reason="gcc with ASan/UBSan runtimes not found")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", lib, SRC, "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = (f"ROOT = {ROOT!r}\nTESTS = {os.path.join(ROOT, 'tests')!r}\nLIB = {lib!r}\n"
            + CHILD)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    report = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, report
    assert "sanitized oracle ok" in r.stdout, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
