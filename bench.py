"""Throughput of the Graph Machine sparse-layer pass on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  gm_ser_forward   A' = Sparsify_4(A A)             (16 two-hop candidates)
  gm_sea_forward   o = SEA(q, k, v, A'), saving p / w per slot and a copy of
                   the unit's edge row (64 B/unit)
  gm_sea_backward  dq, dk, dv, dw' from dout and the saved p / w
  gm_ser_backward  dw (both legs are A, so both contributions land in dw)
on B=8 sequences of n=4096 tokens, 16 query / 8 KV heads, d=128, bf16
activations, fp32 edges and gradients, edges half local (previous 64
tokens) and half far (uniform on [0, i]).  Inputs are resident in HBM
before timing starts; outputs and workspace are preallocated.

Prints one JSON line: units (tokens x KV heads) per second, the pass's
algorithmic HBM bandwidth, per-call times from HIP events on the launch
stream, the roofline entry of the dominant call, and the CPU oracle's rate
on a bounded sample of the same workload (rank 0, N=1: one core, then all
host cores).  The headline is the median cold pass (a 512 MiB scratch write
before each pass evicts the L2s and the MALL) with p10/p90; beside it the
warm pass (back to back), the pass replayed from a HIP graph, and the
pass's counter bytes (calibrated
FETCH_SIZE + WRITE_SIZE from the committed profile, when it matches the
kernel sources) against its compulsory bytes.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-cold]
    python bench.py --config {sea2,ser_sea4,stack21,long64k,theia}   (other workloads)
    python bench.py --config decode   (latency of one decode step)
    python bench.py --config legmix   (leg construction, two legs fwd + bwd)
"""
from __future__ import annotations

import argparse
import json
import statistics
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_dynamic_routing_amd as gm  # noqa: E402
import synth  # noqa: E402

METRIC = ("SER+SEA fwd+bwd tokens·KV-heads/s at n=4096,s1=4; "
          "achieved HBM GB/s vs peak")
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 matrix-core peak (no sparsity)

# Algorithmic (compulsory) bytes per unit: every input byte read once, every
# output byte written once; K/V counted once per unit (unique rows).
# G = 2 query heads per KV head, d = 128, bf16 activations, fp32 gradients;
# the forward's saved p / w (G * s1 fp32) is written once and read once, and
# so is its pair-major copy of the edge row (the backward reads the copy, not
# the edge tensor).
BYTES_PER_UNIT = {
    "gm_ser_forward": 32 + 32 + 8,                      # A row + A' row + path map
    "gm_sea_forward": 512 + 32 + 512 + 512 + 32 + 32,   # q, A', K+V, o, p / w, A' copy
    "gm_sea_backward": 512 + 512 + 32 + 512 + 32 + 1024 + 16 + 1024,
    #                  q    dO  A'copy KV  p/w   dq   dw'   dK dV
    "gm_ser_backward": 32 + 8 + 16 + 16,                # A, path map, dw', dw
}
# with the fused forward (gm_ser_sea_forward): the SER row in, A' and the
# SEA forward's outputs out, no A' read in between
BYTES_PER_UNIT["gm_ser_sea_forward"] = (BYTES_PER_UNIT["gm_ser_forward"] +
                                        BYTES_PER_UNIT["gm_sea_forward"] - 32)
SEPARATE_CALLS = ["gm_ser_forward", "gm_sea_forward", "gm_sea_backward", "gm_ser_backward"]
FUSED_CALLS = ["gm_ser_sea_forward", "gm_sea_backward", "gm_ser_backward"]
CALLS = SEPARATE_CALLS
# The same model without the forward's saved p / w (the pages' path: 5,360
# bytes per unit for the pass, 3,632 for the SEA backward), printed beside
# the line's own figures.
SURVEY_BYTES_PER_UNIT = {"gm_ser_forward": 64, "gm_sea_forward": 1568,
                         "gm_sea_backward": 3632, "gm_ser_backward": 96}
SURVEY_PASS_BYTES_PER_UNIT = sum(SURVEY_BYTES_PER_UNIT.values())
SURVEY_BYTES_PER_UNIT["gm_ser_sea_forward"] = 64 + 1568 - 32
# kernels each call launches on this workload (base names as the profiler
# reports them, template arguments dropped)
CALL_KERNELS = {
    "gm_ser_sea_forward": ["ser_sea_fwd_row_kernel"],
    "gm_ser_forward": ["ser_fwd_vec_kernel"],
    "gm_sea_forward": ["sea_fwd_row_kernel"],
    "gm_sea_backward": ["sea_bwd_src_row_kernel", "edge_index_one_kernel",
                        "sea_bwd_dst_row_s_kernel"],
    "gm_ser_backward": ["ser_bwd_part_kernel", "ser_bwd_part_sum_kernel"],
}
PROFILE = os.path.join(ROOT, "profiles", "metric_pass_kernels.md")

# The other configurations: the stages one step runs (edges carried from one
# SER step to the next), and compulsory bytes per unit of each stage at the
# configuration's slot counts (G = 2, d = 128, bf16 activations).
CONFIG_STAGES = {
    "metric": ["ser_fwd", "sea_fwd", "sea_bwd", "ser_bwd"],
    "sea2": ["sea_fwd"],
    "ser_sea4": ["ser_fwd", "sea_fwd"],
    "stack21": ["ser_fwd", "ser_fwd", "sea_fwd"],   # one of the 21 layers
    "long64k": ["ser_fwd", "sea_fwd", "sea_bwd", "ser_bwd"],
    "theia": ["ser_fwd", "sea_fwd", "sea_bwd", "ser_bwd"],   # (s1, s2, s3) = (2, 4, 4)
    "d64": ["ser_fwd", "sea_fwd", "sea_bwd", "ser_bwd"],     # head dim 64
    "d256": ["ser_fwd", "sea_fwd", "sea_bwd", "ser_bwd"],    # head dim 256
    "fp32": ["ser_fwd", "sea_fwd", "sea_bwd", "ser_bwd"],    # fp32 activations
}


def stage_bytes(stage: str, p: synth.Preset) -> int:
    """Compulsory bytes per unit of one stage (edges: 8 bytes per slot; the
    forward saves p / w, 4 bytes per query head and slot (8 for fp32 inputs,
    whose statistics are fp64), and a copy of the edge row, only when a
    backward follows; the backward reads that copy in place of the edge
    row)."""
    s1 = p.s1
    G = p.hq // p.hkv
    es = 2 if p.dtype == torch.bfloat16 else 4
    qrow, kv = G * p.d * es, 2 * p.d * es          # a unit's q (or o, dout); its K and V rows
    st = (4 if es == 2 else 8) * G * s1 if p.backward else 0
    pm = 8 if p.backward and max(p.s1, p.s2, p.s3) <= 4 else 0   # the SER path map
    return {"ser_fwd": 8 * p.s2 + 8 * s1 + pm,
            "ser_chain2": 8 * p.s2 + 8 * s1,      # A0 in, A2 out; A1 never leaves the chip
            "sea_fwd": qrow + 8 * s1 + kv + qrow + st + (8 * s1 if p.backward else 0),
            "sea_bwd": 2 * qrow + 8 * s1 + kv + st + 4 * G * p.d + 4 * s1 + 8 * p.d,
            "ser_bwd": (8 * p.s2 + pm + 4 * s1 + 4 * p.s2 if pm
                        else 8 * p.s2 + 8 * s1 + 4 * s1 + 4 * p.s2)}[stage]


def profiled_traffic(call: str):
    """Calibrated HBM bytes per launch of `call` from the committed counter
    summary, or None when it is missing or the kernels changed since."""
    from sparse_dynamic_routing_amd.profile_summary import summary_hash_ok
    if not os.path.exists(PROFILE):
        return None
    kernels = {}
    for line in open(PROFILE):
        line = line.strip()
        if line.startswith("kernel:"):
            parts = [x.strip() for x in line.split("|")]
            name = parts[0].split(":", 1)[1].strip()
            kv = dict(x.split("=") for x in parts[1:])
            kernels[name] = float(kv["fetch_bytes"]) + float(kv["write_bytes"])
    if not summary_hash_ok(PROFILE):
        return None
    total = 0.0
    for name in CALL_KERNELS[call]:
        hits = [v for k, v in kernels.items() if k.split("<")[0] == name]
        if len(hits) != 1:
            return None
        total += hits[0]
    return total


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="metric",
                    choices=list(CONFIG_STAGES) + ["decode", "legmix", "refresh"],
                    help="workload: the measured pass (default) or one of the other "
                         "configurations, timed on its own stages (no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="time warm passes only (no flush between passes) and skip the graph "
                         "replay: for profiler runs of the eager pass")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--fused", action="store_true",
                    help="run SER and SEA forward as the one fused call gm_ser_sea_forward "
                         "(measured slower than the two calls on this workload)")
    ap.add_argument("--chain2", action="store_true",
                    help="with --config stack21: the two chained SER steps as the one call "
                         "gm_ser_forward_chain2")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the pass, run a plain device copy of MIB MiB "
                         "(the known-size reference for hardware byte counters)")
    ap.add_argument("--dispatch-probe", action="store_true",
                    help="time the start of 262,144 wavefronts that each store one word per "
                         "lane, as one-wavefront and as four-wavefront workgroups "
                         "(libgm_probe.so; measurement only)")
    ap.add_argument("--gather-probe", action="store_true",
                    help="instead of the pass, measure the 256-byte-row gather ceilings "
                         "(libgm_probe.so) by set size per XCD and loads in flight")
    return ap.parse_args()


# Gather-ceiling probe: sets per XCD (MB) from L2-resident to far beyond the
# caches, 2^20 rows gathered per XCD per launch (2 GB in all).
PROBE_SETS_MB = [1, 2, 3, 4, 6, 8, 16, 64, 256]
PROBE_ROWS_PER_XCD = 1 << 20


def run_gather_probe(a):
    """Median TB/s of 256-byte rows gathered by 16-lane teams (the SEA
    kernels' pattern), per set size per XCD and loads in flight per team."""
    import ctypes
    path = os.path.join(ROOT, "sparse_dynamic_routing_amd", "libgm_probe.so")
    lib = ctypes.CDLL(path)
    f = lib.gm_probe_gather
    f.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    grid = 8 * 256
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    big = max(PROBE_SETS_MB) << 20
    table = torch.ones(8 * big // 4, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda")
    st = torch.cuda.current_stream()
    out = []
    for mb in PROBE_SETS_MB:
        rows = (mb << 20) // 256
        gen.manual_seed(20260902 + mb)
        idx = torch.randint(0, rows, (8, PROBE_ROWS_PER_XCD), generator=gen, device="cuda",
                            dtype=torch.int32)
        for inf in (1, 2, 4):
            def launch():
                rc = f(table.data_ptr(), rows, idx.data_ptr(), PROBE_ROWS_PER_XCD, inf,
                       sink.data_ptr(), grid, st.cuda_stream)
                if rc:
                    raise RuntimeError(f"gm_probe_gather returned {rc}")
            for _ in range(max(a.warmup, 1)):
                launch()
            ts = []
            for _ in range(max(a.steps, 3)):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                launch()
                e1.record(st)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
            t = statistics.median(ts)
            out.append({"set_MB_per_xcd": mb, "in_flight": inf, "us": round(t * 1e6, 1),
                        "TBps": round(8 * PROBE_ROWS_PER_XCD * 256 / t / 1e12, 2)})
            print(json.dumps(out[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"gather_probe": out, "rows_per_xcd_per_launch": PROBE_ROWS_PER_XCD,
                      "row_bytes": 256, "workgroups": grid}))


def run_dispatch_probe(a):
    """Median microseconds to start 262,144 wavefronts (the target pass's
    one per target row at the measured shape) as one- or four-wavefront
    workgroups, each lane storing one word."""
    import ctypes
    path = os.path.join(ROOT, "sparse_dynamic_routing_amd", "libgm_probe.so")
    lib = ctypes.CDLL(path)
    f = lib.gm_probe_dispatch
    f.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    waves = 262144
    out = torch.empty(waves * 64, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    res = {}
    for wpg in (1, 4):
        ts = []
        for it in range(max(a.warmup, 1) + max(a.steps, 5)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            rc = f(out.data_ptr(), waves, wpg, st.cuda_stream)
            e1.record(st)
            e1.synchronize()
            if rc:
                raise RuntimeError(f"gm_probe_dispatch returned {rc}")
            if it >= max(a.warmup, 1):
                ts.append(e0.elapsed_time(e1) * 1e3)
        res[f"{wpg}_wave_workgroups_us"] = round(statistics.median(ts), 1)
    print(json.dumps({"dispatch_probe": res, "waves": waves,
                      "how": "one word stored per lane; HIP events around the launch"}))


class Pass:
    """Device inputs, preallocated outputs and the four calls of one step."""

    def __init__(self, p: synth.Preset):
        self.p = p
        idx, w = synth.edges(p.seed, p.B, p.n, p.hkv, p.s2, mode=p.mode)
        self.host_edges = (idx, w)
        dt = p.dtype
        qs, ks = (p.B, p.n, p.hq, p.d), (p.B, p.n, p.hkv, p.d)
        self.host_act = {name: synth.normal(p.seed, name, shape, dt)
                         for name, shape in (("q", qs), ("k", ks), ("v", ks), ("dout", qs))}
        cu = lambda t: t.contiguous().cuda()  # noqa: E731
        self.idx, self.w = cu(torch.from_numpy(idx)), cu(torch.from_numpy(w))
        self.q, self.k, self.v, self.dout = (cu(self.host_act[n]) for n in ("q", "k", "v", "dout"))
        f32 = dict(dtype=torch.float32, device="cuda")
        es = (p.B, p.n, p.hkv, p.s1)
        self.ia = torch.empty(es, dtype=torch.int32, device="cuda")
        self.wa = torch.empty(es, **f32)
        self.o = torch.empty_like(self.q)
        # p / w per query head and slot, saved by the forward for the backward
        self.stats = (torch.empty(gm.stats_shape(self.q, p.hkv, p.s1), **f32)
                      if p.backward else None)
        self.dq = torch.empty(qs, **f32)
        self.dk = torch.empty(ks, **f32)
        self.dv = torch.empty(ks, **f32)
        self.dwa = torch.empty(es, **f32)
        self.dA = torch.empty(self.idx.shape, **f32)
        # the SER forward's path map, read by the SER backward
        self.paths = (torch.empty(self.idx.shape[:3], dtype=torch.int64, device="cuda")
                      if p.backward and max(p.s1, p.s2, p.s3) <= 4 else None)
        self.ws = gm.ser_workspace(self.idx, self.idx, aliased=True)
        self.ws_sea = gm.sea_workspace(self.q, self.ia)
        if p.ser_steps > 1:   # the first of two chained SER steps writes here
            self.ia1 = torch.empty(es, dtype=torch.int32, device="cuda")
            self.wa1 = torch.empty(es, **f32)

    def stage_calls(self, stages):
        """(label, call) for the stages of one step of a configuration."""
        out, edges = [], (self.idx, self.w)     # edges entering the next SER step
        n_ser = stages.count("ser_fwd")
        for k, st in enumerate(stages):
            if st == "ser_fwd":
                ser_no = stages[:k + 1].count("ser_fwd")
                dst = (self.ia, self.wa) if ser_no == n_ser else (self.ia1, self.wa1)
                src = edges
                # the last SER step's path map feeds the SER backward
                pm = self.paths if ser_no == n_ser else None
                out.append((f"gm_ser_forward#{ser_no}",
                            lambda s_=src, d_=dst, pm_=pm: gm.gm_ser_forward(*s_, *s_, *d_,
                                                                            paths=pm_)))
                edges = dst
            elif st == "ser_chain2":   # two chained SER steps in one launch
                out.append(("gm_ser_forward_chain2",
                            lambda: gm.gm_ser_forward_chain2(self.idx, self.w, self.ia, self.wa)))
                n_ser = 1
                edges = (self.ia, self.wa)
            elif st == "sea_fwd":
                e = (self.ia, self.wa) if n_ser else (self.idx, self.w)
                out.append(("gm_sea_forward",
                            lambda e_=e: gm.gm_sea_forward(self.q, self.k, self.v, *e_, self.o,
                                                           stats=self.stats)))
            elif st == "sea_bwd":
                out.append(("gm_sea_backward", self.calls()[2]))
            else:
                out.append(("gm_ser_backward", self.calls()[3]))
        return out

    def calls(self, fused=False):
        """The step's calls in order, named as in CALLS (FUSED_CALLS with the
        fused forward)."""
        if fused:
            return [
                lambda: gm.gm_ser_sea_forward(self.idx, self.w, self.idx, self.w, self.q,
                                              self.k, self.v, self.ia, self.wa, self.o,
                                              stats=self.stats, paths=self.paths),
            ] + self.calls()[2:]
        return [
            lambda: gm.gm_ser_forward(self.idx, self.w, self.idx, self.w, self.ia, self.wa,
                                      paths=self.paths),
            lambda: gm.gm_sea_forward(self.q, self.k, self.v, self.ia, self.wa, self.o,
                                      stats=self.stats),
            lambda: gm.gm_sea_backward(self.q, self.k, self.v, self.ia, self.wa, self.dout,
                                       self.dq, self.dk, self.dv, self.dwa, self.ws_sea,
                                       stats=self.stats),
            lambda: gm.gm_ser_backward(self.idx, self.w, self.idx, self.w, self.ia, self.wa,
                                       self.dwa, self.dA, self.dA, self.ws, paths=self.paths),
        ]


def time_steps(ps: Pass, steps: int, warmup: int, flush_mib: int = 0, fused: bool = False):
    """Per-step and per-call times (ms, HIP events on the launch stream) of
    `steps` passes after `warmup` untimed ones.  With `flush_mib` > 0 a
    scratch buffer of that many MiB is written before every pass (evicting
    the 4 MB L2s and the 256 MB MALL: a cold pass); only the pass itself lies
    between its events.  The device is synchronised before and after the
    timed steps; returns (per-step ms, {call: per-step ms}, wall seconds)."""
    calls = ps.calls(fused)
    names = FUSED_CALLS if fused else SEPARATE_CALLS
    scratch = (torch.empty(flush_mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
               if flush_mib else None)
    for w in range(warmup):
        if scratch is not None:
            scratch.fill_(float(w))
        for c in calls:
            c()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(steps):
        if scratch is not None:
            scratch.fill_(float(s_ + 1))
        ev[s_][0].record()
        for i, c in enumerate(calls):
            c()
            ev[s_][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [ev[s_][0].elapsed_time(ev[s_][-1]) for s_ in range(steps)]
    per_call = {name: [ev[s_][i].elapsed_time(ev[s_][i + 1]) for s_ in range(steps)]
                for i, name in enumerate(names)}
    del scratch
    return per_step, per_call, wall


def stats_ms(xs):
    """Median, p10, p90 and mean of a list of times."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean())}


def time_graph(ps: Pass, steps: int, fused: bool = False):
    """Mean time of one pass replayed from a HIP graph that captured the
    step's calls (HIP events around `steps` back-to-back replays)."""
    calls = ps.calls(fused)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(steps):
        g.replay()
    en.record()
    torch.cuda.synchronize()
    return st.elapsed_time(en) / steps


def run_config(a):
    """Time one of the other configurations on its own stages (warm, HIP
    events around each stage) and print one JSON line for it."""
    p = synth.PRESETS[a.config]
    stages = CONFIG_STAGES[a.config]
    label = a.config
    if a.chain2:
        if stages[:2] != ["ser_fwd", "ser_fwd"]:
            raise SystemExit(f"--chain2 needs a configuration with two chained SER steps, "
                             f"not {a.config}")
        stages = ["ser_chain2"] + stages[2:]
        label = f"{a.config}_chain2"
    ps = Pass(p)
    calls = ps.stage_calls(stages)
    for _ in range(a.warmup):
        for _, c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(a.steps)]
    for s_ in range(a.steps):
        ev[s_][0].record()
        for i, (_, c) in enumerate(calls):
            c()
            ev[s_][i + 1].record()
    torch.cuda.synchronize()
    per_stage = {lab: float(np.mean([ev[s_][i].elapsed_time(ev[s_][i + 1])
                                     for s_ in range(a.steps)]))
                 for i, (lab, _) in enumerate(calls)}
    ms = float(np.mean([ev[s_][0].elapsed_time(ev[s_][-1]) for s_ in range(a.steps)]))
    U = p.units
    step_bytes = sum(stage_bytes(st, p) for st in stages) * U
    counter = profiled_step_bytes(label)
    print(json.dumps({
        "config": label, "stages": stages, "units_per_step": U,
        "shape": {"B": p.B, "n": p.n, "hq": p.hq, "hkv": p.hkv, "d": p.d,
                  "s1": p.s1, "s2": p.s2, "dtype": str(p.dtype).replace("torch.", "")},
        "ms_per_step": ms, "value": U / (ms * 1e-3), "unit": "tokens·KV-heads/s",
        "per_stage_ms": per_stage,
        "compulsory_bytes_per_unit": step_bytes // U,
        "algorithmic_GBps": step_bytes / (ms * 1e-3) / 1e9,
        "algorithmic_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "counter": None if counter is None else {
            "bytes": counter, "GBps": counter / (ms * 1e-3) / 1e9,
            "frac_of_peak": counter / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "over_compulsory": counter / step_bytes,
            "source": f"profiles/{label}_kernels.md"},
        "steps": a.steps, "warmup": a.warmup, "data": "synthetic"}), flush=True)


def run_decode(a):
    """Latency of one decode step (gm_decode_step) on the metric shape: B = 8
    sequences whose newest token sits at position 4095 of a 4,096-token
    cache, 16 q / 8 KV heads, d = 128, bf16, (s1, s2, s3) = (4, 4, 4), leg 1 =
    the cache's own row of that token.  One JSON line."""
    p = synth.PRESETS["metric"]
    idx, w = synth.edges(p.seed, p.B, p.n, p.hkv, p.s2, mode=p.mode)
    cu = lambda t: t.contiguous().cuda()  # noqa: E731
    idx, w = cu(torch.from_numpy(idx)), cu(torch.from_numpy(w))
    k = cu(synth.normal(p.seed, "k", (p.B, p.n, p.hkv, p.d), p.dtype))
    v = cu(synth.normal(p.seed, "v", (p.B, p.n, p.hkv, p.d), p.dtype))
    q = cu(synth.normal(p.seed, "q", (p.B, p.hq, p.d), p.dtype))
    i1, w1 = idx[:, -1].contiguous(), w[:, -1].contiguous()
    io = torch.empty((p.B, p.hkv, p.s1), dtype=torch.int32, device="cuda")
    wo = torch.empty((p.B, p.hkv, p.s1), dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    step = lambda: gm.gm_decode_step(i1, w1, idx, w, q, k, v, io, wo, o)  # noqa: E731
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(a.steps):
        step()
    en.record()
    torch.cuda.synchronize()
    ms = st.elapsed_time(en) / a.steps
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(16):
            step()
    g.replay()
    torch.cuda.synchronize()
    st.record()
    for _ in range(max(1, a.steps // 16)):
        g.replay()
    en.record()
    torch.cuda.synchronize()
    gms = st.elapsed_time(en) / (max(1, a.steps // 16) * 16)
    print(json.dumps({
        "config": "decode", "units_per_step": p.B * p.hkv, "tokens_per_step": p.B,
        "cache_tokens": p.n, "shape": {"B": p.B, "hq": p.hq, "hkv": p.hkv, "d": p.d,
                                       "s1": p.s1, "s2": p.s2, "s3": p.s3, "dtype": "bfloat16"},
        "us_per_step": ms * 1e3, "tokens_per_s": p.B / (ms * 1e-3),
        "graph_us_per_step": gms * 1e3,
        "how": "back-to-back steps on one stream (HIP events); graph: 16 steps per replay",
        "steps": a.steps, "warmup": a.warmup, "data": "synthetic"}), flush=True)


def run_legmix(a):
    """Leg construction at the metric shape: K = 16 stored edges per unit
    (B = 8, n = 4096, 8 KV heads, local/far mix) mixed into the two legs of
    s = 4 slots the referral composes, forward and backward of both legs.
    One JSON line (per-call times from HIP events)."""
    p = synth.PRESETS["metric"]
    K, s = 16, 4
    idx, w = synth.edges(p.seed, p.B, p.n, p.hkv, K, mode=p.mode)
    rng = np.random.default_rng(p.seed)
    cu = lambda t: torch.from_numpy(t).contiguous().cuda()  # noqa: E731
    idx, w = cu(idx), cu(w)
    alphas = [cu((rng.random((p.hkv, K)) + 0.05).astype(np.float32)) for _ in range(2)]
    shp = (p.B, p.n, p.hkv, s)
    legs = [(torch.empty(shp, dtype=torch.int32, device="cuda"),
             torch.empty(shp, dtype=torch.float32, device="cuda")) for _ in range(2)]
    dleg = cu(rng.standard_normal(shp).astype(np.float32))
    dws = [torch.empty(idx.shape, dtype=torch.float32, device="cuda") for _ in range(2)]
    das = [torch.empty((p.hkv, K), dtype=torch.float32, device="cuda") for _ in range(2)]
    nbytes = gm.gm_leg_mix_backward_workspace_bytes(p.B, p.n, p.hkv, K)
    ws = torch.empty(max(nbytes, 8) // 8, dtype=torch.float64, device="cuda")
    fwd = lambda: [gm.gm_leg_mix_forward(idx, w, alphas[l], *legs[l]) for l in range(2)]  # noqa
    bwd = lambda: [gm.gm_leg_mix_backward(idx, w, alphas[l], *legs[l], dleg, dws[l], das[l],  # noqa
                                          ws) for l in range(2)]
    for _ in range(a.warmup):
        fwd(); bwd()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tf = tb = 0.0
    for _ in range(a.steps):
        e[0].record(); fwd(); e[1].record(); bwd(); e[2].record()
        torch.cuda.synchronize()
        tf += e[0].elapsed_time(e[1]); tb += e[1].elapsed_time(e[2])
    # the same calls replayed from HIP graphs (8 steps per graph): kernel
    # time without the Python launch gaps of the eager loop above
    def graph_us(fn, reps=10, per_graph=8):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / (reps * per_graph) * 1e3
    gf, gb = graph_us(fwd), graph_us(bwd)
    U = p.B * p.n * p.hkv
    fwd_bytes = 2 * (8 * K + 8 * s)                 # both legs: stored row in, leg out
    bwd_bytes = 2 * (8 * K + 12 * s + 4 * K)        # + leg row and dleg in, dw out
    print(json.dumps({
        "config": "legmix", "units_per_step": U, "K": K, "s": s, "legs": 2,
        "forward_us": tf / a.steps * 1e3, "backward_us": tb / a.steps * 1e3,
        "graph_forward_us": gf, "graph_backward_us": gb,
        "units_per_s": U / ((gf + gb) * 1e-6),
        "compulsory_bytes_per_unit": {"forward": fwd_bytes, "backward": bwd_bytes},
        "roofline": {"kernel": "leg_mix_vec_kernel (both legs, graph replay)", "bound": "hbm",
                     "achieved": fwd_bytes * U / (gf * 1e-6) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s",
                     "frac": fwd_bytes * U / (gf * 1e-6) / 1e9 / PEAK_HBM_GBS},
        "steps": a.steps, "warmup": a.warmup, "data": "synthetic"}), flush=True)


def run_refresh(a):
    """Refresh edges from the dense layer of the measured model (B = 8,
    n = 4096, 16 query / 8 KV heads, d = 128, bf16, s = 4): the full call
    (lse pass + selection pass) and the selection alone (lse given, as when
    the dense layer saves its own).  One JSON line; the score contraction is
    priced against the bf16 matrix-core peak."""
    p = synth.PRESETS["metric"]
    s = 4
    seed = synth.BASE_SEED + 40
    q = synth.normal(seed, "q", (p.B, p.n, p.hq, p.d), torch.bfloat16, 0, "cuda")
    k = synth.normal(seed, "k", (p.B, p.n, p.hkv, p.d), torch.bfloat16, 0, "cuda")
    shp = (p.B, p.n, p.hkv, s)
    io = torch.empty(shp, dtype=torch.int32, device="cuda")
    wo = torch.empty(shp, dtype=torch.float32, device="cuda")
    lse = torch.empty((p.B, p.n, p.hq), dtype=torch.float32, device="cuda")
    full = lambda: gm.gm_dense_refresh(q, k, lse, io, wo)  # noqa: E731
    sel = lambda: gm.gm_dense_refresh(q, k, lse, io, wo, lse_given=True)  # noqa: E731
    for _ in range(a.warmup):
        full(); sel()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tf = ts = 0.0
    for _ in range(a.steps):
        e[0].record(); full(); e[1].record(); sel(); e[2].record()
        torch.cuda.synchronize()
        tf += e[0].elapsed_time(e[1]); ts += e[1].elapsed_time(e[2])
    tf, ts = tf / a.steps, ts / a.steps
    # the same query width with one query head per KV head (hq = hkv = 16):
    # G = 1 takes the one-pass kernel (lse and the edges together)
    k1 = synth.normal(seed, "k", (p.B, p.n, p.hq, p.d), torch.bfloat16, 0, "cuda")
    io1 = torch.empty((p.B, p.n, p.hq, s), dtype=torch.int32, device="cuda")
    wo1 = torch.empty((p.B, p.n, p.hq, s), dtype=torch.float32, device="cuda")
    full1 = lambda: gm.gm_dense_refresh(q, k1, lse, io1, wo1)  # noqa: E731
    sel1 = lambda: gm.gm_dense_refresh(q, k1, lse, io1, wo1, lse_given=True)  # noqa: E731
    for _ in range(a.warmup):
        full1(); sel1()
    torch.cuda.synchronize()
    tf1 = ts1 = 0.0
    for _ in range(a.steps):
        e[0].record(); full1(); e[1].record(); sel1(); e[2].record()
        torch.cuda.synchronize()
        tf1 += e[0].elapsed_time(e[1]); ts1 += e[1].elapsed_time(e[2])
    tf1, ts1 = tf1 / a.steps, ts1 / a.steps
    pairs = p.B * p.hq * p.n * (p.n + 1) // 2          # causal (token, key, query head)
    flops = 2 * p.d * pairs                            # one score contraction
    print(json.dumps({
        "config": "refresh", "B": p.B, "n": p.n, "hq": p.hq, "hkv": p.hkv, "d": p.d, "s": s,
        "full_us": tf * 1e3, "select_us": ts * 1e3, "lse_pass_us": (tf - ts) * 1e3,
        "tokens_per_s": p.B * p.n / (tf * 1e-3),
        "score_flops_per_pass": flops,
        "select_tflops": flops / (ts * 1e-3) / 1e12, "mfma_peak_tflops": PEAK_BF16_TFLOPS,
        "scores_per_s": pairs / (ts * 1e-3),
        "mha_g1": {"hq": p.hq, "hkv": p.hq, "one_pass_us": tf1 * 1e3,
                   "select_alone_us": ts1 * 1e3,
                   "one_pass_tflops": flops / (tf1 * 1e-3) / 1e12,
                   "how": "G = 1: one launch forms lse and keeps the top scores"},
        "roofline": {"kernel": "refresh_kernel (selection pass)", "bound": "mfma",
                     "achieved": flops / (ts * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops / (ts * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "steps": a.steps, "warmup": a.warmup, "data": "synthetic"}), flush=True)


def profiled_step_bytes(config: str):
    """Counter bytes per step from profiles/<config>_kernels.md, or None when
    it is missing or the kernel sources changed since."""
    from sparse_dynamic_routing_amd.profile_summary import summary_hash_ok
    path = os.path.join(ROOT, "profiles", f"{config}_kernels.md")
    if not os.path.exists(path):
        return None
    per_step = None
    for line in open(path):
        line = line.strip()
        if line.startswith("bytes_per_step:"):
            per_step = float(line.split(":", 1)[1])
    return per_step if summary_hash_ok(path) else None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host_threads() -> int:
    """Threads for the all-cores leg: the cores this process may run on,
    at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(ps: Pass, budget_s: float):
    """The oracle as it stands (single-threaded C in fp64) on whole (batch, KV
    head) pairs of the same workload: first on one core, pairs in order until
    `budget_s` is spent; then on all host cores, the same functions on
    disjoint pairs from a pool of threads (every stage is local to a pair;
    the C calls release the interpreter lock), whole rounds of all pairs
    until `budget_s` is spent.  The all-cores rate is the reported value."""
    import concurrent.futures as cf
    import oracle
    orc = oracle.get()
    p = ps.p
    G = p.hq // p.hkv
    idx, w = ps.host_edges
    act = {k: v.float().numpy() for k, v in ps.host_act.items()}
    pairs = [(b, h) for b in range(p.B) for h in range(p.hkv)]

    def one_pair(bh):
        b, h = bh
        sl = lambda x, g=0: np.ascontiguousarray(  # noqa: E731
            x[b:b + 1, :, h * g:(h + 1) * g] if g else x[b:b + 1, :, h:h + 1])
        e_i, e_w = sl(idx), sl(w).astype(np.float64)
        q, k, v, do = (np.ascontiguousarray(sl(act[n], G if n in ("q", "dout") else 0),
                                            dtype=np.float64) for n in ("q", "k", "v", "dout"))
        ia, wa = orc.ser_forward(e_i, e_w, e_i, e_w, p.s1)
        orc.sea_forward(q, k, v, ia, wa)
        dq, dk, dv, dwa = orc.sea_backward(q, k, v, ia, wa, do)
        orc.ser_backward(e_i, e_w, e_i, e_w, ia, wa, dwa, aliased=True)

    done, spent = 0, 0.0
    while spent < budget_s and done < 16 * len(pairs):
        t0 = time.perf_counter()
        one_pair(pairs[done % len(pairs)])
        spent += time.perf_counter() - t0
        done += 1
    one_rate = done * p.n / spent

    nthr = _host_threads()
    rounds, mspent = 0, 0.0
    with cf.ThreadPoolExecutor(max_workers=nthr) as ex:
        while mspent < budget_s and rounds < 16:
            t0 = time.perf_counter()
            list(ex.map(one_pair, pairs))
            mspent += time.perf_counter() - t0
            rounds += 1
    all_units = rounds * len(pairs) * p.n
    all_rate = all_units / mspent
    return {"value": all_rate, "unit": "tokens·KV-heads/s", "cores": nthr, "kind": "oracle",
            "sample": f"{rounds} rounds of all {len(pairs)} (batch, KV head) pairs of the "
                      f"measured workload ({all_units} units, {mspent:.1f} s) on {nthr} "
                      f"threads, each thread running the single-threaded C oracle (fp64) on "
                      f"whole pairs",
            "cpu_model": _cpu_model(),
            "single_core": {"value": one_rate, "cores": 1,
                            "sample": f"{done} whole pairs ({done * p.n} units, "
                                      f"{spent:.1f} s) in order on one thread"},
            "speedup_over_one_core": all_rate / one_rate}


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no cross-GPU step (units are "
              "independent per (batch, KV head)); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        n = a.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(a.warmup + a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                          "launches": a.warmup + a.steps}))
        return
    if a.gather_probe:
        run_gather_probe(a)
        return
    if a.dispatch_probe:
        run_dispatch_probe(a)
        return
    gm.load()
    if a.config == "decode":
        run_decode(a)
        return
    if a.config == "legmix":
        run_legmix(a)
        return
    if a.config == "refresh":
        run_refresh(a)
        return
    if a.config != "metric":
        run_config(a)
        return
    p = synth.PRESETS["metric"]
    ps = Pass(p)
    torch.cuda.synchronize()
    U = p.units
    # headline: cold passes (a 512 MiB write before each evicts L2s and MALL),
    # median over the timed steps; warm (back-to-back) passes beside it
    fused = a.fused
    calls_used = FUSED_CALLS if fused else SEPARATE_CALLS
    cold_steps, cold_calls, wall = time_steps(ps, a.steps, a.warmup,
                                              flush_mib=0 if a.no_cold else 512, fused=fused)
    warm_steps, warm_calls, _ = time_steps(ps, a.steps, a.warmup, fused=fused)
    cold, warm = stats_ms(cold_steps), stats_ms(warm_steps)
    ms = cold["median"]
    per_call = {c: stats_ms(v)["median"] for c, v in cold_calls.items()}
    graph_ms = None if a.no_cold else time_graph(ps, a.steps, fused=fused)
    pass_bytes = sum(BYTES_PER_UNIT[c] for c in calls_used) * U
    survey_pass_bytes = SURVEY_PASS_BYTES_PER_UNIT * U
    dom = max(per_call, key=per_call.get)
    traffic = {c: profiled_traffic(c) for c in calls_used}
    counter_bytes = (sum(traffic.values()) if all(v is not None for v in traffic.values())
                     else None)
    dom_gbs = BYTES_PER_UNIT[dom] * U / (per_call[dom] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": U / (ms * 1e-3),
        "unit": "tokens·KV-heads/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "SER+SEA layer pass fwd+bwd: B=8, n=4096, 16 q / 8 KV heads, "
                               "d=128, s1=s2=s3=4, local/far edge mix",
                   "B": p.B, "n": p.n, "hq": p.hq, "hkv": p.hkv, "d": p.d,
                   "s1": p.s1, "s2": p.s2, "s3": p.s3, "units_per_step": U,
                   "parallelism": "single GPU"},
        "calls": calls_used,
        "timing": ("cold" if not a.no_cold else "warm") +
                  ": median over the timed steps of HIP events around each pass"
                  + (" (512 MiB written before each pass, outside its events)"
                     if not a.no_cold else ""),
        "ms_per_step_p10_p90": [cold["p10"], cold["p90"]],
        "pass_algorithmic_GBps": pass_bytes / (ms * 1e-3) / 1e9,
        "pass_frac_of_peak": pass_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "pass_frac_of_peak_at_5360_B_per_unit":
            survey_pass_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "per_call_ms": per_call,
        "warm": {"ms_per_step": warm["median"], "p10": warm["p10"], "p90": warm["p90"],
                 "mean": warm["mean"], "value": U / (warm["median"] * 1e-3),
                 "per_call_ms": {c: stats_ms(v)["median"] for c, v in warm_calls.items()},
                 "how": "the same passes back to back, no flush"},
        "cold_mean_ms": cold["mean"],
        "graph": None if graph_ms is None else {
            "ms_per_step": graph_ms, "value": U / (graph_ms * 1e-3),
            "how": "the four calls captured once in a HIP graph, replayed back to back (warm)"},
        "pass_counter": None if counter_bytes is None else {
            "bytes": counter_bytes,
            "GBps": counter_bytes / (ms * 1e-3) / 1e9,
            "frac_of_peak": counter_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "over_compulsory": counter_bytes / pass_bytes,
            "source": "profiles/metric_pass_kernels.md (calibrated FETCH_SIZE + WRITE_SIZE)"},
        "roofline": {"kernel": dom, "kernels": CALL_KERNELS[dom], "bound": "hbm",
                     "achieved": dom_gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": dom_gbs / PEAK_HBM_GBS,
                     "traffic": traffic[dom],
                     "bytes_per_unit": BYTES_PER_UNIT[dom], "units_per_launch": U,
                     "frac_at_survey_bytes": (SURVEY_BYTES_PER_UNIT.get(dom, BYTES_PER_UNIT[dom])
                                              * U / (per_call[dom] * 1e-3) / 1e9 / PEAK_HBM_GBS),
                     "survey_bytes_per_unit": SURVEY_BYTES_PER_UNIT.get(dom)},
        "wall_s_timed": wall,
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(ps, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
