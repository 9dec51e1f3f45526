"""The C ABI's host-side argument checks built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only: every `-fsanitize` is passed
through `-Xarch_host`, the device code is built as usual) and driven by the
argument-check tests of test_abi.py, in a child process with clang's ASan
runtime preloaded.  None of these calls reaches a kernel launch, so no GPU
is needed; any out-of-bounds access or undefined behaviour in the checks
aborts the child.

Building the whole library takes a minute or two of hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from sparse_dynamic_routing_amd import build as gmbuild  # noqa: E402

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

CHILD = textwrap.dedent("""
    import inspect, sys
    sys.path.insert(0, ROOT)
    sys.path.insert(0, TESTS)
    from sparse_dynamic_routing_amd import binding
    lib = binding.load(LIB)
    import test_abi
    ran = 0
    for name, f in inspect.getmembers(test_abi, inspect.isfunction):
        if name.startswith("test_") and list(inspect.signature(f).parameters) == ["lib"]:
            f(lib)
            ran += 1
    print("sanitized checks ok", ran)
""")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not os.path.exists(gmbuild.HIPCC) or _asan_runtime() is None,
                    reason="hipcc or clang's ASan runtime not found")
def test_argument_checks_under_host_sanitizers(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([gmbuild.HIPCC, *gmbuild.FLAGS,
                            *gmbuild.FILE_FLAGS.get(os.path.basename(src), []), *HOST_SAN,
                            "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, gmbuild.sources()))
    lib = str(tmp_path / "libgm_san.so")
    r = subprocess.run([gmbuild.HIPCC, f"--offload-arch={gmbuild.ARCH}", "-shared", "-fPIC",
                        "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = (f"ROOT = {ROOT!r}\nTESTS = {os.path.join(ROOT, 'tests')!r}\nLIB = {lib!r}\n"
            + CHILD)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    report = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, report
    assert "sanitized checks ok" in r.stdout, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    shutil.rmtree(tmp_path, ignore_errors=True)
