"""Benchmark of the KDA chunked forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--seg-chunks L]
                    [--no-cpu-baseline] [--no-variants] [--no-bwd]
    python bench.py --write-traffic WORKLOAD FETCH_CSV WRITE_CSV [--stats-csv CSV] [--counters-csv CSV ...]

Workload: the 8192-token prefill, B=1, T=8192, H=32 (q/k and value heads),
K=V=128, chunk 64, bf16 I/O, h0 = 0, seeded synthetic inputs (synth/).  A step is
one kda_fwd call (the whole hot path: the intra-chunk kernel, then the state scan's
kernels) on inputs already resident in HBM.  Prints one JSON line.

Timing.  W warmup steps, continued for at least --settle-s seconds so that the GPU
clocks have ramped up.  The headline (value, ms_per_step) is cold-cache: each of
the K timed steps follows a 1 GiB read through the caches, which evicts the 4 MB
L2s and the 256 MB MALL, and is timed alone by two HIP events on the call's stream
(created with hipEventDisableSystemFence, so recording one costs no system-scope
cache flush).  The whole timed region, flushes included, sits between two device
synchronizations.  The warm rate (back-to-back steps, wall clock) and the split
into the intra call and the scan call (events around every fourth warm step) are
reported as well.

Algorithmic bytes per token and value head (K = V = 128): q, k, g, v, o at 256 B
each plus beta 2 B = 1,282 B (q, k per q/k head), plus h0 read and ht written once
per (sequence, head).  The intra kernel necessarily reads q, k, g, beta (770 B); the
scan reads v and writes o (512 B) and ht.  Algorithmic flops per token and head:
180,224 (dense 64-row tiles).  `roofline` is the whole call: algorithmic bytes over
the cold call time, against the HBM peak; `traffic` is the call's HBM bytes from
the committed rocprofv3 FETCH_SIZE / WRITE_SIZE counters (profiles/), null once a
kernel's source has changed since they were taken.  `kernels` lists each kernel of
the call with its necessary bytes, counter bytes and rocprofv3 average duration.

The backward's reverse state scan (kda_bwd_dhu) is timed on the same shape as a
separate object (``bwd_dhu``), in the checkpoint format of the bwd_dhu page (bf16
dhc, fp32 dht / dh0).  Its algorithmic bytes per token and value head: qg, kg, w
read (768 B), do and dv read (512 B), dv2 written (256 B); per chunk and head the
decay row (K fp32) read and the checkpoint (K x V bf16) written; dht read and dh0
written once per (sequence, head).  Its inputs are synthetic stand-ins with the
forward operands' shapes and magnitudes, built on the device outside the timed
region (the scan's time does not depend on the values).

--write-traffic turns the CSV output of two rocprofv3 --pmc runs (FETCH_SIZE, then
WRITE_SIZE) of this script into profiles/traffic_counters.json for WORKLOAD, scaled
by what the counters read for the 256 MiB device copy the script makes; with
--stats-csv also the per-kernel average durations of a --kernel-trace --stats run,
with --counters-csv the per-kernel medians of further counter runs (SQ counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
CFG_ID = 3
METRIC = "KDA fwd tokens/s at T=8192,H=32,K=V=128 bf16; % of HBM/MFMA roofline"
FLOPS_PER_TOKEN_HEAD = 180224
# Sources whose change invalidates a kernel's committed counter figures.  The scan
# kernels include the host header that chooses between them (a figure taken on one
# scan must not be reported for a call that now runs the other).
_CS = "gated_delta_rule_chunked_amd/csrc/"
_SCAN = [_CS + "kda_scan.hip", _CS + "kda_device.hpp", _CS + "kda_plan.hpp"]
KERNEL_SOURCES = {
    "prep": [_CS + "kda_intra.hip"],
    "chunk_table": [_CS + "kda_intra.hip"],
    "intra": [_CS + "kda_intra.hip", _CS + "kda_device.hpp"],
    "inter": [_CS + "kda_inter.hip", _CS + "kda_device.hpp", _CS + "kda_plan.hpp"],
    "bwd_dhu": [_CS + "kda_bwd.hip", _CS + "kda_device.hpp"],
    "bscan_state": [_CS + "kda_bwd_scan.hip", _CS + "kda_device.hpp", _CS + "kda_plan.hpp"],
    "bscan_full": [_CS + "kda_bwd_scan.hip", _CS + "kda_device.hpp", _CS + "kda_plan.hpp"],
    "scan_state": _SCAN,
    "scan_full": _SCAN,
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hip_runtime_api.h
CALIB_BYTES = 256 << 20       # the device copy whose counters calibrate FETCH_SIZE / WRITE_SIZE


class HipEvents:
    """Timing events of the HIP runtime that torch (and libkda) already loaded,
    created with hipEventDisableSystemFence: recording one then costs no system-scope
    cache write-back and invalidation, which torch's default events pay (several us
    per record on MI355X, inflating the steps they bracket)."""

    def __init__(self, n):
        import ctypes
        self._c = ctypes
        hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        vp = ctypes.c_void_p
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [vp, vp]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        hip.hipEventDestroy.argtypes = [vp]
        self._hip = hip
        self.ev = []
        for _ in range(n):
            e = vp()
            st = hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
            if st != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed with status {st}")
            self.ev.append(e)

    def record(self, i, stream):
        st = self._hip.hipEventRecord(self.ev[i], self._c.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed with status {st}")

    def ms(self, i, j):
        """Milliseconds from event i to event j (both complete)."""
        f = self._c.c_float()
        st = self._hip.hipEventElapsedTime(self._c.byref(f), self.ev[i], self.ev[j])
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed with status {st}")
        return f.value

    def __del__(self):
        for e in getattr(self, "ev", []):
            self._hip.hipEventDestroy(e)


def algorithmic_bytes(d):
    """(intra bytes, inter bytes) per call, as defined in the module docstring."""
    B, T, HQK, HV, K, V, N = (d[x] for x in ("B", "T", "HQK", "HV", "K", "V", "N"))
    intra = B * T * (2 * HQK * K * 2 + HV * K * 2 + HV * 2)
    inter = B * T * HV * V * 2 * 2 + N * HV * K * V * 4 * (1 + (d["h0"] is not None))
    return intra, inter


def _code_only(text):
    """C++ source without comments and blank space, so that editing a comment does not
    invalidate a kernel's counter figures (string literals in these files hold no
    comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(_code_only(open(os.path.join(ROOT, f)).read()).encode())
    return h.hexdigest()[:16]


def kernel_key(name):
    """Short key of a library kernel from its demangled name ("void kda::scan_full_kernel<128,
    false>(kda::Params, int)" -> "scan_full"; chunk-16 instances get "_c16"), else None."""
    import re
    base = name.split("(")[0].replace("void ", "").strip()
    m = re.match(r"kda::(\w+?)_kernel(?:<\d+(?:, (true|false))?>)?$", base)
    if not m:
        return None
    return m.group(1) + ("_c16" if m.group(2) == "true" else "")


def _source_key(key):
    return key[:-4] if key.endswith("_c16") else key


def load_traffic(workload):
    try:
        return json.load(open(TRAFFIC_FILE))["workloads"][workload]
    except (OSError, KeyError, ValueError):
        return None


def kernel_figures(workload, keys):
    """Committed counter figures of these kernels for the workload: {key: entry or None}.
    An entry measured on another version of the kernel's source is dropped (None)."""
    w = load_traffic(workload) or {}
    out = {}
    for k in keys:
        t = w.get(k)
        out[k] = t if t is not None and t.get("source_sha") == source_sha(_source_key(k)) else None
    return out


def traffic_for(workload, keys):
    """HBM bytes per call (the sum over the call's kernels), or None when a kernel's
    figures are missing or stale."""
    figs = kernel_figures(workload, keys)
    if any(v is None or "bytes_per_launch" not in v for v in figs.values()):
        return None
    return sum(v["bytes_per_launch"] for v in figs.values())


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(d, budget_s=18.0):
    """The fp64 oracle as it stands, on bounded samples of the workload (all heads, the
    first tokens of the sequence): O1, the token recurrence (numpy, one thread), and O2,
    the chunked form at chunk 64 (numpy and scipy with every host core given to BLAS).
    Each sample grows by threes until a run takes a thirtieth of the budget, then jumps to the
    size that should take a third of it, so the two timed samples take about 12 s together.
    The headline value is the faster of the two, as tokens/s of the whole layer."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import chunked, recurrent
    host_cores = len(os.sched_getaffinity(0))

    def timed(fn, threads, n0, cap):
        n = n0
        with threadpool_limits(limits=threads):
            while True:
                a = {k: d[k][:, :n] for k in ("q", "k", "v", "g", "beta")}
                t0 = time.perf_counter()
                fn(**a, scale=d["scale"])
                dt = time.perf_counter() - t0
                if dt > budget_s / 6 or n >= cap:
                    return n, dt
                # a run this long predicts the rate well enough to size the timed one
                n = min(cap, int(n * budget_s / 3 / dt) if dt > budget_s / 30 else n * 3)

    n1, t1 = timed(recurrent, 1, 64, d["T"])
    n2, t2 = timed(chunked, host_cores, 64, d["T"])
    blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    o1 = {"tokens_per_s": n1 / t1, "threads": 1, "tokens": n1, "seconds": t1,
          "what": "token recurrence (O1), numpy fp64, vectorised over heads, serial over tokens"}
    o2 = {"tokens_per_s": n2 / t2, "threads": host_cores, "tokens": n2, "seconds": t2,
          "what": "chunked form at chunk 64 (O2), numpy/scipy fp64, exact per-element gates, BLAS threads = host cores"}
    best = o1 if o1["tokens_per_s"] >= o2["tokens_per_s"] else o2
    return {"value": best["tokens_per_s"], "unit": "tokens/s", "cores": best["threads"], "kind": "oracle",
            "sample": f"first {best['tokens']} tokens x {d['HV']} heads of the workload, {best['what']}, "
                      f"{best['seconds']:.1f} s; tokens/s of the full {d['HV']}-head layer",
            "o1": o1, "o2": o2, "host_cores": host_cores, "cpu_model": cpu_model(), "blas": blas}


def bwd_algorithmic_bytes(B, T, HV, K, V, N, C):
    """Bytes one kda_bwd_dhu call must move (bf16 checkpoints, fp32 dht / dh0)."""
    return (B * T * HV * (3 * K * 2 + 3 * V * 2)     # qg, kg, w; do, dv, dv2
            + C * HV * (K * 4 + K * V * 2)          # decay row, checkpoint
            + 2 * N * HV * K * V * 4)               # dht, dh0


def bwd_kernels(plan, nt):
    """Keys of the kernels one fixed-length kda_bwd_dhu call launches.  The backward picks its
    scan with the forward's rule on the same shape: `plan` is kda_fwd_scan_plan at chunk 64."""
    if plan == 0:
        return ["bwd_dhu"]
    return (["bscan_state"] if plan < nt else []) + ["bscan_full"]


def bench_bwd(t, d, dev, stream, steps, workload, keys, seg_chunks=0):
    """Time kda_bwd_dhu at the workload's shape; returns the bwd_dhu object.  `keys` names the
    kernels one call launches (their summed counter bytes are the object's traffic)."""
    import torch
    from gated_delta_rule_chunked_amd import KDA_FLAG_CKPT_BF16, kda_bwd_dhu_raw, make_bwd_args, num_chunks
    B, T, HV, K, V, N = d["B"], d["T"], d["HV"], d["K"], d["V"], d["N"]
    NT = (T + 63) // 64
    gen = torch.Generator(device=dev)
    gen.manual_seed(33)
    # chunk-local cumsum of g in log2 units (T is a multiple of 64 here)
    g = t["g"].float().reshape(B, NT, 64, HV, K)
    g2 = (torch.cumsum(g, dim=2) * 1.4426950408889634).reshape(B, T, HV, K).contiguous()
    last = g2.reshape(B, NT, 64, HV, K)[:, :, 63:].expand(B, NT, 64, HV, K).reshape(B, T, HV, K)
    qh = t["q"].float().repeat_interleave(HV // d["HQK"], dim=2)
    kh = t["k"].float().repeat_interleave(HV // d["HQK"], dim=2)
    qg = (qh * torch.exp2(g2)).to(torch.bfloat16)
    kg = (kh * torch.exp2(last - g2)).to(torch.bfloat16)
    w = (kh * torch.exp2(g2) * t["beta"].float()[..., None]).to(torch.bfloat16)
    do = torch.randn((B, T, HV, V), generator=gen, device=dev).to(torch.bfloat16)
    dv = (0.1 * torch.randn((B, T, HV, V), generator=gen, device=dev)).to(torch.bfloat16)
    dht = 0.1 * torch.randn((N, HV, K, V), generator=gen, device=dev)
    C = num_chunks(T, None, B)
    dv2 = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=dev)
    dh0 = torch.empty((N, HV, K, V), dtype=torch.float32, device=dev)
    dhc = torch.empty((C, HV, K, V), dtype=torch.bfloat16, device=dev)
    a = make_bwd_args(qg, kg, w, g2, do, dv, dht, d["scale"], None, dv2, dh0, dhc, stream=stream.cuda_stream,
                      flags=KDA_FLAG_CKPT_BF16, seg_chunks=seg_chunks)
    from gated_delta_rule_chunked_amd import kda_bwd_dhu_workspace_bytes
    ws = torch.empty(max(kda_bwd_dhu_workspace_bytes(a), 256), dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    for _ in range(3):
        kda_bwd_dhu_raw(a)
    torch.cuda.synchronize()
    ev = HipEvents(steps + 1)   # call i runs between events i and i + 1
    for i in range(steps):
        ev.record(i, stream)
        kda_bwd_dhu_raw(a)
    ev.record(steps, stream)
    torch.cuda.synchronize()
    ms = float(np.mean([ev.ms(i, i + 1) for i in range(steps)]))
    nbytes = bwd_algorithmic_bytes(B, T, HV, K, V, N, C)
    achieved = nbytes / (ms * 1e-3) / 1e9
    flops = 6 * K * V * B * T * HV       # DV, QD, WD per token and head
    return {"ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "algorithmic_bytes": nbytes,
            "kernels": keys,
            "roofline": {"bound": "hbm", "kernel": "bwd_dhu", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": traffic_for(workload, keys)},
            "mfma_frac": flops / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
            "checkpoints": "bf16", "states": "fp32", "data": "synthetic stand-ins for qg, kg, w, g2, do, dv, dht"}


def write_traffic(workload, fetch_csv, write_csv, stats_csv=None, counter_csvs=()):
    """profiles/traffic_counters.json entry for `workload` from rocprofv3 --pmc output
    (run_counter_collection.csv of a FETCH_SIZE run and of a WRITE_SIZE run of this
    script): per library kernel the median over its dispatches of each counter (KiB),
    scaled by the ratio of the 256 MiB copy's bytes to what the counter read for it (the
    copy dispatch with the largest value); with stats_csv (run_kernel_stats.csv of a
    --kernel-trace --stats run) also each kernel's average duration; with counter_csvs
    (further --pmc runs) each kernel's median per dispatch of every counter in them,
    summed over the counter's instances."""
    import collections
    import csv
    import statistics

    def per_dispatch(path):
        val, name = collections.defaultdict(float), {}
        for r in csv.DictReader(open(path)):
            val[r["Dispatch_Id"]] += float(r["Counter_Value"])
            name[r["Dispatch_Id"]] = r["Kernel_Name"]
        return val, name

    f, fn = per_dispatch(fetch_csv)
    w, wn = per_dispatch(write_csv)
    cf = max(v for k, v in f.items() if "copyBuffer" in fn[k])
    cw = max(v for k, v in w.items() if "copyBuffer" in wn[k])
    ff, wf = CALIB_BYTES / (cf * 1024), CALIB_BYTES / (cw * 1024)
    ent = {"calibration": {"copy_bytes": CALIB_BYTES, "copy_fetch_kib": cf, "copy_write_kib": cw,
                           "fetch_factor": ff, "write_factor": wf}}
    acc = collections.defaultdict(lambda: [[], []])
    for k, v in f.items():
        key = kernel_key(fn[k])
        if key:
            acc[key][0].append(v)
    for k, v in w.items():
        key = kernel_key(wn[k])
        if key:
            acc[key][1].append(v)
    for key, (fv, wv) in acc.items():
        if not fv or not wv:
            continue
        fk, wk = statistics.median(fv), statistics.median(wv)
        ent[key] = {"source_sha": source_sha(_source_key(key)), "fetch_kib": fk, "write_kib": wk,
                    "fetch_bytes": fk * 1024 * ff, "write_bytes": wk * 1024 * wf,
                    "bytes_per_launch": fk * 1024 * ff + wk * 1024 * wf}
    for path in counter_csvs:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        vals = collections.defaultdict(lambda: collections.defaultdict(list))
        for did, cs in per.items():
            key = kernel_key(names[did])
            if key:
                for c, v in cs.items():
                    vals[key][c].append(v)
        for key, cs in vals.items():
            ent.setdefault(key, {"source_sha": source_sha(_source_key(key))})
            ent[key].setdefault("counters", {}).update({c: statistics.median(v) for c, v in cs.items()})
    if stats_csv:
        for r in csv.DictReader(open(stats_csv)):
            key = kernel_key(r["Name"])
            if key:
                ent.setdefault(key, {"source_sha": source_sha(_source_key(key))})
                ent[key]["rocprof_calls"] = int(r["Calls"])
                ent[key]["rocprof_avg_us"] = float(r["AverageNs"]) / 1e3
    try:
        out = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        out = {"workloads": {}}
    out["note"] = ("HBM bytes per launch: FETCH_SIZE x fetch_factor + WRITE_SIZE x write_factor (KiB), factors "
                   "from a 256 MiB device copy in the same run; medians over launches; rocprof_avg_us from "
                   "rocprofv3 --kernel-trace --stats of the default bench command")
    out["workloads"][workload] = ent
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(ent, indent=1))


def call_kernels(plan, nt, varlen, c16=False):
    """Keys of the kernels one kda_fwd call launches: the chunk table (varlen) or the
    counter reset, the intra kernel, then the serial scan, or the segmented scan's
    passes (the state pass only when a sequence can have several segments: segment
    length `plan` below the chunk count `nt` of the longest possible sequence)."""
    sfx = "_c16" if c16 else ""
    keys = ["chunk_table" if varlen else "prep", "intra" + sfx]
    if plan == 0:
        keys.append("inter")
    else:
        if plan < nt:   # some sequence has several segments
            keys.append("scan_state" + sfx)
        keys.append("scan_full" + sfx)
    return keys


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed cold-cache steps (the headline)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-steps", type=int, default=100, help="back-to-back steps for the warm rate")
    ap.add_argument("--event-every", type=int, default=4,
                    help="time the two calls of every n-th warm step with events (each record costs ~2.5 us)")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="keep warming up until this many seconds have passed (GPU clocks ramp up under load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip timing the forward's options")
    ap.add_argument("--no-bwd", action="store_true", help="skip timing the backward state scan")
    ap.add_argument("--config", type=int, default=CFG_ID, choices=sorted(range(1, 6)),
                    help="workload (synth/inputs.py CONFIGS); the headline metric is quoted on 3")
    ap.add_argument("--seg-chunks", type=int, default=0,
                    help="segment length of the state scan (0: the library's choice)")
    ap.add_argument("--chunk", type=int, default=64, choices=(16, 64), help="chunk length of the timed call")
    ap.add_argument("--write-traffic", nargs=3, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--stats-csv", default=None)
    ap.add_argument("--counters-csv", nargs="*", default=[])
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, stats_csv=args.stats_csv, counter_csvs=args.counters_csv)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_chunked_amd import (alloc_workspace, kda_fwd_inter, kda_fwd_intra, kda_fwd_raw,
                                              kda_fwd_scan_plan, load_library, make_args, max_chunks)
    from synth import make_config_inputs
    from synth.inputs import CONFIGS

    load_library()
    dev = torch.device("cuda:0")
    d = make_config_inputs(args.config)
    t = {k: torch.from_numpy(d[k]).to(torch.bfloat16).to(dev) for k in ("q", "k", "v", "g", "beta")}
    h0 = None if d["h0"] is None else torch.from_numpy(d["h0"]).to(dev)
    cu = None if d["cu_seqlens"] is None else torch.from_numpy(d["cu_seqlens"]).to(dev)
    B, T, HV, K, V, N = d["B"], d["T"], d["HV"], d["K"], d["V"], d["N"]
    o = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((N, HV, K, V), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    a = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], h0, cu, o, ht,
                  stream=stream.cuda_stream, seg_chunks=args.seg_chunks, chunk=args.chunk)
    ws = alloc_workspace(a, dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    plan = kda_fwd_scan_plan(a)   # 0: 16-column serial scan; else 64-column segments of `plan` chunks
    nt = (T + 63) // 64

    # plain copy of known size: the byte-counter calibration kernel for rocprofv3 --pmc
    calib_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)

    def step():
        kda_fwd_raw(a)

    # W warmup steps, continued until the clocks have settled (--settle-s of steps)
    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t0 < args.settle_s:
        step()
        n_warm += 1
        if n_warm % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # ---- headline: K cold-cache steps.  A 1 GiB buffer is read through the caches
    # before each (evicting L2 and MALL; read, not written, so that no dirty lines are
    # left whose write-back the step would pay), then the step alone is timed by events.
    flush = torch.ones(1 << 27, dtype=torch.int64, device=dev)
    cev = HipEvents(2 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush.sum()
        cev.record(2 * i, stream)
        step()
        cev.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    region_wall = time.perf_counter() - t0
    cold = np.array([cev.ms(2 * i, 2 * i + 1) for i in range(args.steps)])
    del flush
    ms_per_step = float(cold.mean())

    # ---- warm: back-to-back steps (wall clock); every --event-every-th step is run as its
    # two calls with events before the intra call, before the scan call and after it
    t_end = time.perf_counter() + 0.3   # clocks settle again after the cold-cache steps
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    sampled = list(range(0, args.warm_steps, max(1, args.event_every)))
    ev = HipEvents(3 * len(sampled))
    slot = {i: j for j, i in enumerate(sampled)}
    t0 = time.perf_counter()
    for i in range(args.warm_steps):
        j = slot.get(i)
        if j is None:
            step()
            continue
        ev.record(3 * j, stream)
        kda_fwd_intra(a)
        ev.record(3 * j + 1, stream)
        kda_fwd_inter(a)
        ev.record(3 * j + 2, stream)
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3 / args.warm_steps
    intra_ms = np.array([ev.ms(3 * j, 3 * j + 1) for j in range(len(sampled))])
    inter_ms = np.array([ev.ms(3 * j + 1, 3 * j + 2) for j in range(len(sampled))])

    # the box's device-copy bandwidth (bytes read + written per second), for context
    cpy = HipEvents(2)
    cpy.record(0, stream)
    for _ in range(5):
        calib_dst.copy_(calib_src)
    cpy.record(1, stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * calib_src.numel() / (cpy.ms(0, 1) * 1e-3) / 1e9

    # the forward's options, same workload, warm back-to-back calls (informational)
    variants_ms = None
    if not args.no_variants:
        from gated_delta_rule_chunked_amd import KDA_FLAG_BETA_LOGITS, KDA_FLAG_STATE_BF16
        variants_ms = {}
        ht_bf = torch.empty((N, HV, K, V), dtype=torch.bfloat16, device=dev)
        hc = torch.empty((max_chunks(T, N, B, cu is not None), HV, K, V), dtype=torch.float32, device=dev)
        # the plain call first, timed the same way, as the control for the options
        for name, kw in (("plain", dict(flags=0, ht=ht)),
                         ("beta_logits", dict(flags=KDA_FLAG_BETA_LOGITS, ht=ht)),
                         ("bf16_state", dict(flags=KDA_FLAG_STATE_BF16, ht=ht_bf)),
                         ("chunk_states_fp32", dict(flags=0, ht=ht, hc=hc)),
                         ("chunk16", dict(flags=0, ht=ht, chunk=16))):
            ht_v = kw.pop("ht")
            h0v = None if h0 is None else h0.to(ht_v.dtype)
            av = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], h0v, cu, o, ht_v,
                           stream=stream.cuda_stream, seg_chunks=args.seg_chunks, **kw)
            av.workspace, av.workspace_bytes = ws.data_ptr(), ws.numel()
            t_end = time.perf_counter() + 0.3
            while time.perf_counter() < t_end:
                for _ in range(20):
                    kda_fwd_raw(av)
                torch.cuda.synchronize()
            vev = HipEvents(2)
            vev.record(0, stream)
            for _ in range(20):
                kda_fwd_raw(av)
            vev.record(1, stream)
            torch.cuda.synchronize()
            variants_ms[name] = vev.ms(0, 1) / 20
        del hc, ht_bf

    # the backward's stand-in operands are built for fixed-length, whole-chunk sequences
    workload = CONFIGS[args.config].name + (f"_seg{args.seg_chunks}" if args.seg_chunks else "") + \
        ("_chunk16" if args.chunk == 16 else "")
    bwd = None
    if not args.no_bwd and d["cu_seqlens"] is None and d["T"] % 64 == 0:
        a64 = type(a).from_buffer_copy(a)
        a64.chunk = 64
        bwd = bench_bwd(t, d, dev, stream, args.steps, workload, bwd_kernels(kda_fwd_scan_plan(a64), nt),
                        seg_chunks=args.seg_chunks)

    tokens = B * T
    value = tokens / (ms_per_step * 1e-3)
    ab_intra, ab_scan = algorithmic_bytes(d)
    path_bytes = ab_intra + ab_scan
    flops = FLOPS_PER_TOKEN_HEAD * tokens * HV
    keys = call_kernels(plan, nt, cu is not None, args.chunk == 16)
    figs = kernel_figures(workload, keys)
    traffic = traffic_for(workload, keys)
    achieved = path_bytes / (ms_per_step * 1e-3) / 1e9
    necessary = {"intra": ab_intra, "inter": ab_scan, "scan_full": ab_scan}
    kernels = []
    for k in keys:
        f = figs[k] or {}
        row = {"kernel": k, "necessary_bytes": necessary.get(_source_key(k), 0),
               "counter_bytes": f.get("bytes_per_launch"), "rocprof_avg_us": f.get("rocprof_avg_us")}
        if row["rocprof_avg_us"]:   # this kernel's own fraction: its necessary bytes over its average duration
            row["achieved_GBs"] = row["necessary_bytes"] / (row["rocprof_avg_us"] * 1e-6) / 1e9
            row["frac_of_hbm_peak"] = row["achieved_GBs"] / HBM_PEAK_GBS
            if row["counter_bytes"]:
                row["traffic_TBs"] = row["counter_bytes"] / (row["rocprof_avg_us"] * 1e-6) / 1e12
        kernels.append(row)
    timed = [r for r in kernels if r["rocprof_avg_us"]]
    if timed:   # the kernel with the longest average duration
        max(timed, key=lambda r: r["rocprof_avg_us"])["dominant"] = True
    calls = {}
    for name, arr, nb in (("intra", intra_ms, ab_intra), ("scan", inter_ms, ab_scan)):
        m = float(arr.mean())
        calls[name] = {"ms": m, "necessary_bytes": nb, "achieved_GBs": nb / (m * 1e-3) / 1e9,
                       "frac_of_hbm_peak": nb / (m * 1e-3) / (HBM_PEAK_GBS * 1e9)}
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CONFIGS[args.config].name, "B": B, "T": T, "N": d["N"], "HQK": d["HQK"], "HV": HV,
                   "K": K, "V": V, "chunk": args.chunk, "h0": "zero" if d["h0"] is None else "0.1 N(0,1)",
                   "varlen": d["cu_seqlens"] is not None, "seg_chunks": args.seg_chunks,
                   "scan": "16-column serial" if plan == 0 else f"64-column, segments of {plan} chunks"},
        "timing": "cold cache: each timed step follows a 1 GiB read through L2 and MALL and is timed alone "
                  "with HIP events; ms_per_step is their mean",
        "step_ms_p10_p50_p90": [float(x) for x in np.percentile(cold, [10, 50, 90])],
        "timed_region_wall_ms": region_wall * 1e3,
        "roofline": {"bound": "hbm", "kernel": "kda_fwd call (" + ", ".join(keys) + ")", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": path_bytes},
        "kernels": kernels,
        "calls_warm": calls,
        "warm": {"ms_per_step": warm_ms, "tokens_per_s": tokens / (warm_ms * 1e-3),
                 "hbm_frac": path_bytes / (warm_ms * 1e-3) / (HBM_PEAK_GBS * 1e9)},
        "path_roofline": {"algorithmic_bytes": path_bytes, "algorithmic_flops": flops,
                          "hbm_frac": path_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                          "mfma_frac": flops / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12)},
        "device_copy_GBs": copy_gbs,
        "options_ms_per_step_warm": variants_ms,
        "bwd_dhu": bwd,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
