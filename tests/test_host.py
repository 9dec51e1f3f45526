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


def test_stats_helpers_read_both_layouts():
    """The saved statistics hold fp32 p / w (bf16 inputs) or fp64 p / w (fp32
    inputs, two words each); the helpers give them per query head, and the
    edge copy, from either layout."""
    B, hkv, n, G, s1 = 2, 2, 5, 3, 3
    q16 = torch.zeros(B, n, hkv * G, 8, dtype=torch.bfloat16)
    q32 = torch.zeros(B, n, hkv * G, 8, dtype=torch.float32)
    assert gm.stats_shape(q16, hkv, s1) == (B, hkv, n, G + 2, s1)
    assert gm.stats_shape(q32, hkv, s1) == (B, hkv, n, 2 * G + 2, s1)
    g = torch.Generator().manual_seed(5)
    pw = torch.rand(B, hkv, n, G, s1, dtype=torch.float64, generator=g)
    idx = torch.randint(0, 5, (B, hkv, n, s1), dtype=torch.int32, generator=g)
    w = torch.rand(B, hkv, n, s1, generator=g)
    want = pw.permute(0, 2, 1, 3, 4).reshape(B, n, hkv * G, s1)
    for E in (1, 2):
        st = torch.zeros(B, hkv, n, E * G + 2, s1)
        flat = st.view(B, hkv, n, (E * G + 2) * s1)
        if E == 1:
            flat[..., :G * s1] = pw.float().reshape(B, hkv, n, G * s1)
        else:
            flat[..., :2 * G * s1] = pw.reshape(B, hkv, n, G * s1).contiguous().view(
                torch.float32).reshape(B, hkv, n, 2 * G * s1)
        st[:, :, :, E * G] = idx.view(torch.float32)
        st[:, :, :, E * G + 1] = w
        got = gm.stats_as_query_heads(st, G)
        assert got.dtype == (torch.float32 if E == 1 else torch.float64)
        assert torch.equal(got.double(), want.float().double() if E == 1 else want)
        ei, ew = gm.stats_edge_copy(st)
        assert torch.equal(ei, idx.permute(0, 2, 1, 3)) and torch.equal(ew, w.permute(0, 2, 1, 3))
    with pytest.raises(ValueError):
        gm.stats_as_query_heads(torch.zeros(B, hkv, n, 7, s1), 3)
