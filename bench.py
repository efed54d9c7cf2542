"""Benchmark of the KDA chunked forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--config N] [--seg-chunks L]

Workload: the 8192-token prefill, B=1, T=8192, H=32 (q/k and value heads),
K=V=128, chunk 64, bf16 I/O, h0 = 0, seeded synthetic inputs (synth/).
A step is one call of the whole hot path (intra-chunk kernel, then the
inter-chunk state scan) on inputs already resident in HBM.  Prints one JSON line.

Algorithmic bytes per token and value head (K = V = 128): q, k, g, v, o at 256 B
each plus beta 2 B = 1,282 B (q, k per q/k head), plus the final state ht once per
(sequence, head).  The intra kernel necessarily reads q, k, g, beta (770 B); the
inter kernel reads v and writes o (512 B) and ht.  Algorithmic flops per token
and head: 180,224 (dense 64-row tiles).

The backward's reverse state scan (kda_bwd_dhu) is timed on the same shape as a
separate object (``bwd_dhu``), in the checkpoint format of the bwd_dhu page (bf16
dhc, fp32 dht / dh0).  Its algorithmic bytes per token and value head: qg, kg, w
read (768 B), do and dv read (512 B), dv2 written (256 B); per chunk and head the
decay row (K fp32) read and the checkpoint (K x V bf16) written; dht read and dh0
written once per (sequence, head).  Its inputs are synthetic stand-ins with the
forward operands' shapes and magnitudes, built on the device outside the timed
region (the scan's time does not depend on the values).
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
KERNEL_SOURCES = {
    "intra": ["gated_delta_rule_chunked_amd/csrc/kda_intra.hip", "gated_delta_rule_chunked_amd/csrc/kda_device.hpp"],
    "inter": ["gated_delta_rule_chunked_amd/csrc/kda_inter.hip", "gated_delta_rule_chunked_amd/csrc/kda_device.hpp"],
    "bwd_dhu": ["gated_delta_rule_chunked_amd/csrc/kda_bwd.hip", "gated_delta_rule_chunked_amd/csrc/kda_device.hpp"],
    "scan_state": ["gated_delta_rule_chunked_amd/csrc/kda_scan.hip", "gated_delta_rule_chunked_amd/csrc/kda_device.hpp"],
    "scan_full": ["gated_delta_rule_chunked_amd/csrc/kda_scan.hip", "gated_delta_rule_chunked_amd/csrc/kda_device.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def algorithmic_bytes(d):
    """(intra bytes, inter bytes) per call, as defined in the module docstring."""
    B, T, HQK, HV, K, V, N = (d[x] for x in ("B", "T", "HQK", "HV", "K", "V", "N"))
    intra = B * T * (2 * HQK * K * 2 + HV * K * 2 + HV * 2)
    inter = B * T * HV * V * 2 * 2 + N * HV * K * V * 4 * (1 + (d["h0"] is not None))
    return intra, inter


def source_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(workload, call):
    """HBM bytes per call from the committed rocprofv3 counter summary: the sum over
    the kernels the call launched for this workload ("intra"; the scan call is the
    serial scan or the segmented scan's passes), or None when the workload is missing
    or any of its kernels was measured on a different version of its source."""
    kernels = {"intra": ["intra"], "inter": ["inter", "scan_state", "scan_full"], "bwd_dhu": ["bwd_dhu"]}[call]
    try:
        w = json.load(open(TRAFFIC_FILE))["workloads"][workload]
    except (OSError, KeyError, ValueError):
        return None
    found = [w[k] for k in kernels if k in w]
    if not found or any(t.get("source_sha") != source_sha(k) for k, t in zip([k for k in kernels if k in w], found)):
        return None
    return sum(t["bytes_per_launch"] for t in found)


def cpu_baseline(d, budget_s=12.0):
    """The fp64 oracle (token recurrence) on a bounded sample: all heads, the
    first tokens of the sequence, grown until about budget_s of CPU work."""
    from threadpoolctl import threadpool_limits
    from oracle import recurrent
    n = 32
    with threadpool_limits(limits=1):
        while True:
            a = {k: d[k][:, :n] for k in ("q", "k", "v", "g", "beta")}
            t0 = time.perf_counter()
            recurrent(**a, scale=d["scale"])
            dt = time.perf_counter() - t0
            if dt > budget_s / 4 or n >= d["T"]:
                break
            n = min(d["T"], n * 4)
    tok_heads_per_s = n * d["HV"] / dt
    return {"value": tok_heads_per_s / d["HV"], "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} tokens x {d['HV']} heads of the workload, fp64 token recurrence "
                      f"(numpy, 1 thread), {dt:.1f} s; tokens/s of the full {d['HV']}-head layer"}


def bwd_algorithmic_bytes(B, T, HV, K, V, N, C):
    """Bytes one kda_bwd_dhu call must move (bf16 checkpoints, fp32 dht / dh0)."""
    return (B * T * HV * (3 * K * 2 + 3 * V * 2)     # qg, kg, w; do, dv, dv2
            + C * HV * (K * 4 + K * V * 2)          # decay row, checkpoint
            + 2 * N * HV * K * V * 4)               # dht, dh0


def bench_bwd(t, d, dev, stream, steps, workload):
    """Time kda_bwd_dhu at the workload's shape; returns the bwd_dhu object."""
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
                      flags=KDA_FLAG_CKPT_BF16)
    for _ in range(3):
        kda_bwd_dhu_raw(a)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        kda_bwd_dhu_raw(a)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    nbytes = bwd_algorithmic_bytes(B, T, HV, K, V, N, C)
    achieved = nbytes / (ms * 1e-3) / 1e9
    flops = 6 * K * V * B * T * HV       # DV, QD, WD per token and head
    return {"ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "algorithmic_bytes": nbytes,
            "roofline": {"bound": "hbm", "kernel": "bwd_dhu", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": traffic_for(workload, "bwd_dhu")},
            "mfma_frac": flops / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
            "checkpoints": "bf16", "states": "fp32", "data": "synthetic stand-ins for qg, kg, w, g2, do, dv, dht"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip timing the forward's options")
    ap.add_argument("--cold", type=int, default=20, help="extra cold-cache steps (flush between)")
    ap.add_argument("--no-bwd", action="store_true", help="skip timing the backward state scan")
    ap.add_argument("--config", type=int, default=CFG_ID, choices=sorted(range(1, 6)),
                    help="workload (synth/inputs.py CONFIGS); the headline metric is quoted on 3")
    ap.add_argument("--seg-chunks", type=int, default=0,
                    help="segment length of the state scan (0: the library's choice)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_chunked_amd import (alloc_workspace, kda_fwd_inter, kda_fwd_intra, load_library,
                                              make_args)
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
                  stream=stream.cuda_stream, seg_chunks=args.seg_chunks)
    ws = alloc_workspace(a, dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()

    # plain copy of known size: the byte-counter calibration kernel for rocprofv3 --pmc
    calib_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        kda_fwd_intra(a)
        if ev is not None:
            ev[1].record(stream)
        kda_fwd_inter(a)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    intra_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    inter_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    ms_per_step = wall * 1e3 / args.steps

    # cold-cache steps: a 1 GiB buffer written between steps evicts L2 and MALL
    cold_ms = None
    if args.cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(args.cold):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        cold_ms = float(np.median(cold))
        del flush

    # the forward's options, same workload (informational; not the headline)
    variants_ms = None
    if not args.no_variants:
        from gated_delta_rule_chunked_amd import KDA_FLAG_BETA_LOGITS, KDA_FLAG_STATE_BF16, num_chunks
        variants_ms = {}
        ht_bf = torch.empty((N, HV, K, V), dtype=torch.bfloat16, device=dev)
        hc = torch.empty((num_chunks(T, cu, B), HV, K, V), dtype=torch.float32, device=dev)
        for name, kw in (("beta_logits", dict(flags=KDA_FLAG_BETA_LOGITS, ht=ht)),
                         ("bf16_state", dict(flags=KDA_FLAG_STATE_BF16, ht=ht_bf)),
                         ("chunk_states_fp32", dict(flags=0, ht=ht, hc=hc))):
            ht_v = kw.pop("ht")
            h0v = None if h0 is None else h0.to(ht_v.dtype)
            av = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], h0v, cu, o, ht_v,
                           stream=stream.cuda_stream, seg_chunks=args.seg_chunks, **kw)
            av.workspace, av.workspace_bytes = ws.data_ptr(), ws.numel()
            for _ in range(2):
                kda_fwd_intra(av)
                kda_fwd_inter(av)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                kda_fwd_intra(av)
                kda_fwd_inter(av)
            e1.record(stream)
            torch.cuda.synchronize()
            variants_ms[name] = e0.elapsed_time(e1) / 10
        del hc, ht_bf

    # the backward's stand-in operands are built for fixed-length, whole-chunk sequences
    bwd = None
    if not args.no_bwd and d["cu_seqlens"] is None and d["T"] % 64 == 0:
        bwd = bench_bwd(t, d, dev, stream, args.steps, CONFIGS[args.config].name)

    tokens = B * T
    value = tokens / (ms_per_step * 1e-3)
    ab_intra, ab_inter = algorithmic_bytes(d)
    kern = {"intra": (float(intra_ms.mean()), ab_intra), "inter": (float(inter_ms.mean()), ab_inter)}
    dom = max(kern, key=lambda k: kern[k][0])
    dom_ms, dom_bytes = kern[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    workload = CONFIGS[args.config].name + (f"_seg{args.seg_chunks}" if args.seg_chunks else "")
    traffic = traffic_for(workload, dom)
    path_bytes = ab_intra + ab_inter
    flops = FLOPS_PER_TOKEN_HEAD * tokens * HV
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CONFIGS[args.config].name, "B": B, "T": T, "N": d["N"], "HQK": d["HQK"], "HV": HV,
                   "K": K, "V": V, "chunk": 64, "h0": "zero" if d["h0"] is None else "0.1 N(0,1)",
                   "varlen": d["cu_seqlens"] is not None, "seg_chunks": args.seg_chunks},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "kernels_ms": {"intra": kern["intra"][0], "inter": kern["inter"][0]},
        "path_roofline": {"algorithmic_bytes": path_bytes,
                          "hbm_frac": path_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                          "mfma_frac": flops / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12)},
        "cold_cache_ms_per_step": cold_ms,
        "options_ms_per_step": variants_ms,
        "bwd_dhu": bwd,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
