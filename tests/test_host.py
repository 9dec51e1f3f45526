"""Host-side behaviour that needs no GPU: the benchmark's one-GPU contract,
the binding's tensor checks, and the profile summaries' link to the sources."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest
import torch

import sparse_dynamic_routing_amd as gm
from sparse_dynamic_routing_amd import profile_summary

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_binding_rejects_host_tensors_before_any_launch():
    idx = torch.zeros((1, 4, 1, 2), dtype=torch.int32)
    w = torch.zeros((1, 4, 1, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        gm.gm_ser_forward(idx, w, idx, w, idx.clone(), w.clone())
    q = torch.zeros((1, 4, 2, 16), dtype=torch.bfloat16)
    k = torch.zeros((1, 4, 1, 16), dtype=torch.bfloat16)
    lse = torch.zeros((1, 4, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        gm.gm_dense_refresh(q, k, lse, idx.clone(), w.clone())


def test_committed_profiles_name_their_command_and_sources():
    """Every committed kernel summary states the command that made it; the
    ones with counter bytes carry the hash of the kernel sources they were
    taken on (bench.py ignores their bytes when the sources changed since)."""
    pdir = os.path.join(ROOT, "profiles")
    names = sorted(f for f in os.listdir(pdir) if f.endswith(".md"))
    assert "metric_pass_kernels.md" in names
    for f in names:
        text = open(os.path.join(pdir, f)).read()
        assert "rocprofv3" in text and "bench.py" in text, f
        if "bytes_per_step:" in text:
            assert "source_hash:" in text, f
    h = profile_summary.source_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)
    assert profile_summary.source_hash(profile_summary.PASS_SOURCES) != h


def test_summary_hash_names_its_sources(tmp_path):
    """A summary is valid while the sources it names hash as recorded; a
    wrong hash, or none, makes it stale."""
    files = profile_summary.PASS_SOURCES
    good = tmp_path / "good.md"
    good.write_text(f"source_files: {','.join(files)}\n"
                    f"source_hash: {profile_summary.source_hash(files)}\n")
    assert profile_summary.summary_hash_ok(str(good))
    bad = tmp_path / "bad.md"
    bad.write_text(f"source_files: {','.join(files)}\nsource_hash: 0123456789abcdef\n")
    assert not profile_summary.summary_hash_ok(str(bad))
    whole = tmp_path / "whole.md"
    whole.write_text(f"source_hash: {profile_summary.source_hash()}\n")
    assert profile_summary.summary_hash_ok(str(whole))
    none = tmp_path / "none.md"
    none.write_text("nothing here\n")
    assert not profile_summary.summary_hash_ok(str(none))


def test_source_hash_ignores_comments_only():
    """A comment edit leaves the code text (and so the profiles' hash) as it
    is; a code edit, or a comment marker inside a string, does not."""
    ct = profile_summary.code_text
    a = 'int f(int x) {  // twice\n    return 2 * x; /* doubled */ }\n'
    b = '// header\nint f(int x) {\n  return 2 * x;\n}'
    assert ct(a) == ct(b)
    assert ct(a) != ct(a.replace("2 * x", "3 * x"))
    s = 'const char* m = "a // b"; // tail'
    assert '"a // b"' in ct(s) and "tail" not in ct(s)
    assert ct('x = 1; /* multi\nline */ y = 2;') == "x = 1; y = 2;"
