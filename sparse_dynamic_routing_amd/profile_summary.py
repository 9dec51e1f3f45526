"""Turn rocprofv3 CSV output of the measured pass into a short summary.

    python -m sparse_dynamic_routing_amd.profile_summary \\
        --trace KT_DIR --fetch FETCH_DIR --write WRITE_DIR \\
        --copy-fetch CFETCH_DIR --copy-write CWRITE_DIR --copy-mib 512 \\
        --command "..." > summary.md

KT_DIR holds a ``--kernel-trace --stats`` run, FETCH_DIR / WRITE_DIR single
counter runs (FETCH_SIZE, WRITE_SIZE) of the same program, CFETCH_DIR /
CWRITE_DIR the same counters for a plain copy of a known size (bench.py
--copy-calibration).  Counters are in KiB per dispatch; each is divided by
what it reads for the copy per byte actually moved, so the byte figures are
calibrated HBM-side bytes.  The summary ends with a machine-readable block
that bench.py reads, including a hash of the kernel sources the numbers
belong to.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)


def code_text(src: str) -> str:
    """C/HIP source without its comments and with runs of whitespace folded,
    so that editing a comment does not change what the hash says was
    measured.  String literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


# The sources the layer pass's kernels are built from (the C ABI, the
# shared headers, SER, SEA and the reverse edge index); a summary names the
# files its hash covers, so work on an unrelated kernel leaves it valid.
PASS_SOURCES = ["edge_index.hip", "gm_api.hip", "gm_common.h", "gm_internal.h", "gm_select.h",
                "gm_wave.h", "sea_bwd.hip", "sea_fwd.hip", "ser.hip"]


def source_hash(files=None) -> str:
    """sha256 over the code (comments left out) of the given csrc files (by
    default every HIP source and header) and the C header: what the counters
    measured."""
    h = hashlib.sha256()
    if files is None:
        paths = sorted(glob.glob(os.path.join(PKG, "csrc", "*")))
    else:
        paths = [os.path.join(PKG, "csrc", f) for f in sorted(files)]
    for f in paths + [os.path.join(ROOT, "include", "gm.h")]:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def summary_hash_ok(path: str) -> bool:
    """True when the summary at `path` carries the hash of the sources it
    names (or of all sources, for a summary that names none) as they are
    now."""
    hsh, files = None, None
    for line in open(path):
        line = line.strip()
        if line.startswith("source_hash:"):
            hsh = line.split(":", 1)[1].strip()
        elif line.startswith("source_files:"):
            files = [f.strip() for f in line.split(":", 1)[1].split(",") if f.strip()]
    return hsh is not None and hsh == source_hash(files)


def short(name: str) -> str:
    name = re.sub(r"gm::\(anonymous namespace\)::", "", name)
    name = re.sub(r"\(.*$", "", name)
    return re.sub(r"^void ", "", name).strip()


def _csv(d: str, suffix: str):
    files = glob.glob(os.path.join(d, f"*{suffix}"))
    if not files:
        raise FileNotFoundError(f"no *{suffix} in {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def kernel_stats(d: str):
    """Calls and average microseconds of this library's kernels (those in
    namespace gm; torch's input draws are left out)."""
    out = {}
    for r in _csv(d, "kernel_stats.csv"):
        if "gm::" in r["Name"]:
            out[short(r["Name"])] = (int(r["Calls"]), float(r["AverageNs"]) / 1000.0)
    return out


def counter(d: str, name: str):
    acc = defaultdict(list)
    for r in _csv(d, "counter_collection.csv"):
        if r["Counter_Name"] == name:
            acc[short(r["Kernel_Name"])].append(float(r["Counter_Value"]) * 1024.0)
    return {k: sum(v) / len(v) for k, v in acc.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--title", default="the measured layer pass")
    ap.add_argument("--workload", default="B=8, n=4096, 16 q / 8 KV heads, d=128, "
                    "s1=s2=s3=4, bf16 activations\n(one SER fwd + SEA fwd + SEA bwd + "
                    "SER bwd per step)")
    ap.add_argument("--sources", default=",".join(PASS_SOURCES),
                    help="csrc files the measured kernels are built from (comma list)")
    ap.add_argument("--steps-run", type=int, default=0,
                    help="passes the profiled program ran (to turn launches into launches "
                         "per pass); default: the fewest launches of any kernel, every kernel "
                         "running at least once per pass")
    a = ap.parse_args()

    ks = kernel_stats(a.trace)
    passes = a.steps_run or min(calls for calls, _ in ks.values())
    fetch, write = counter(a.fetch, "FETCH_SIZE"), counter(a.write, "WRITE_SIZE")
    cf, cw = counter(a.copy_fetch, "FETCH_SIZE"), counter(a.copy_write, "WRITE_SIZE")
    copy_bytes = a.copy_mib * (1 << 20)
    cname = max(cf, key=lambda k: cf[k])          # the copy kernel reads the most
    f_scale = cf[cname] / copy_bytes
    w_scale = cw[cname] / copy_bytes
    print(f"# Kernel durations and HBM traffic of {a.title}\n")
    print(f"Workload: {a.workload}.\n")
    print(f"Command (kernel trace): `{a.command}`\n")
    print(f"Counter runs: the same command with `--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`;"
          f" calibration: `python3 bench.py --copy-calibration {a.copy_mib} --steps 5"
          f" --warmup 0` under the same two counters.\n")
    print(f"Calibration ({cname}, {a.copy_mib} MiB read and written): FETCH_SIZE reads "
          f"{f_scale:.3f} x the bytes read, WRITE_SIZE {w_scale:.3f} x the bytes written; "
          "the byte columns below are divided by these factors.\n")
    print("| kernel | calls | avg us | fetch MB/launch | write MB/launch | GB/s (calibrated) |")
    print("|---|---:|---:|---:|---:|---:|")
    rows = []
    for k, (calls, us) in sorted(ks.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        fb = fetch.get(k, 0.0) / f_scale
        wb = write.get(k, 0.0) / w_scale
        gbs = (fb + wb) / (us * 1e-6) / 1e9 if us else 0.0
        rows.append((k, calls, us, fb, wb))
        print(f"| {k} | {calls} | {us:.1f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {gbs:.0f} |")
    print("\n```")
    files = [f for f in a.sources.split(",") if f]
    print(f"source_files: {','.join(files)}")
    print(f"source_hash: {source_hash(files)}")
    print(f"fetch_scale: {f_scale:.6f}")
    print(f"write_scale: {w_scale:.6f}")
    per_step = 0.0
    for k, calls, us, fb, wb in rows:
        print(f"kernel: {k} | us={us:.3f} | fetch_bytes={fb:.0f} | write_bytes={wb:.0f}")
        per_step += (fb + wb) * calls / passes
    print(f"bytes_per_step: {per_step:.0f}")
    print("```")


if __name__ == "__main__":
    main()
