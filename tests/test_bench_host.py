"""bench.py's host-side arithmetic, on the CPU: the algorithmic bytes and flops it divides
by (against the closed forms of the workloads), the kernel keys it reads from rocprofv3
names, the kernels it attributes to one call, and the counter scaling that turns
FETCH_SIZE / WRITE_SIZE into bytes (on synthetic counter files, written to a temporary
counter file, never to the committed one)."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_of_the_benchmarked_workload():
    d = dict(B=1, T=8192, HQK=32, HV=32, K=128, V=128, N=1, h0=None)
    intra, scan = bench.algorithmic_bytes(d)
    # q, k, g at 256 B and beta at 2 B per token and head; v and o at 256 B; ht once per head
    assert intra == 8192 * 32 * (256 + 256 + 256 + 2)
    assert scan == 8192 * 32 * (256 + 256) + 32 * 128 * 128 * 4
    assert intra + scan == 338_165_760
    # grouped heads: q and k count once per q/k head; an initial state is read once more
    g = dict(d, HQK=16, h0=object())
    gi, gs = bench.algorithmic_bytes(g)
    assert gi == 8192 * (16 * 512 + 32 * 258) and gs == scan + 32 * 128 * 128 * 4


def test_flops_per_token_and_head():
    C, K, V = 64, 128, 128
    # Akk, Aqk and w contract over K; u and the intra output over the chunk; the
    # three state products over K x V
    assert bench.FLOPS_PER_TOKEN_HEAD == 3 * 2 * C * K + 2 * 2 * C * V + 3 * 2 * K * V == 180_224


def test_backward_algorithmic_bytes():
    n = bench.bwd_algorithmic_bytes(B=1, T=8192, HV=32, K=128, V=128, N=1, C=128)
    per_token = 3 * 128 * 2 + 3 * 128 * 2          # qg, kg, w; do, dv, dv2
    per_chunk = 128 * 4 + 128 * 128 * 2             # decay row, bf16 checkpoint
    assert n == 8192 * 32 * per_token + 128 * 32 * per_chunk + 2 * 32 * 128 * 128 * 4 == 543_162_368


@pytest.mark.parametrize("name,key", [
    ("void kda::intra_kernel<128, false>(kda::Params, int, int const*, HIP_vector_type<int, 2u> const*)", "intra"),
    ("void kda::intra_kernel<64, true>(kda::Params, int, int const*, HIP_vector_type<int, 2u> const*)", "intra_c16"),
    ("void kda::scan_full_kernel<128, false>(kda::Params, int)", "scan_full"),
    ("void kda::scan_state_kernel<128, true>(kda::Params, int)", "scan_state_c16"),
    ("kda::prep_kernel(kda::Params)", "prep"),
    ("void kda::bscan_state_kernel<128>(kda::BwdParams, int)", "bscan_state"),
    ("void kda::bwd_dhu_kernel<64>(kda::BwdParams, int)", "bwd_dhu"),
    ("__amd_rocclr_copyBuffer", None),
    ("void at::native::elementwise_kernel<128, 4>(int)", None),
])
def test_kernel_keys(name, key):
    assert bench.kernel_key(name) == key


def test_kernels_of_one_call():
    assert bench.call_kernels(0, 128, False) == ["prep", "intra", "inter"]
    assert bench.call_kernels(32, 128, False) == ["prep", "intra", "scan_state", "scan_full"]
    assert bench.call_kernels(128, 128, True) == ["chunk_table", "intra", "scan_full"]
    assert bench.call_kernels(32, 128, False, c16=True) == ["prep", "intra_c16", "scan_state_c16", "scan_full_c16"]
    assert bench.bwd_kernels(0, 128) == ["bwd_dhu"]
    assert bench.bwd_kernels(32, 128) == ["bscan_state", "bscan_full"]
    assert bench.bwd_kernels(128, 128) == ["bscan_full"]


def _pmc_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_counter_scaling_and_staleness(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy = "__amd_rocclr_copyBuffer"
    intra = "void kda::intra_kernel<128, false>(kda::Params, int, int const*, HIP_vector_type<int, 2u> const*)"
    full = "void kda::scan_full_kernel<128, false>(kda::Params, int)"
    # the 256 MiB copy reads half its bytes in FETCH_SIZE (factor 2) and all of them in
    # WRITE_SIZE (factor 1); counters are summed over instances, medians over dispatches
    fetch = [(1, copy, "FETCH_SIZE", 65536), (1, copy, "FETCH_SIZE", 65536),
             (2, intra, "FETCH_SIZE", 50), (2, intra, "FETCH_SIZE", 50),
             (3, intra, "FETCH_SIZE", 300), (4, intra, "FETCH_SIZE", 200), (5, full, "FETCH_SIZE", 10)]
    write = [(1, copy, "WRITE_SIZE", 262144), (2, intra, "WRITE_SIZE", 7), (3, intra, "WRITE_SIZE", 9),
             (4, intra, "WRITE_SIZE", 8), (5, full, "WRITE_SIZE", 4)]
    _pmc_csv(tmp_path / "f.csv", fetch)
    _pmc_csv(tmp_path / "w.csv", write)
    with open(tmp_path / "s.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs"])
        w.writeheader()
        w.writerow({"Name": intra, "Calls": 3, "AverageNs": 101500.0})
    bench.write_traffic("wl", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), stats_csv=str(tmp_path / "s.csv"))
    ent = json.load(open(tmp_path / "traffic.json"))["workloads"]["wl"]
    assert ent["calibration"]["fetch_factor"] == pytest.approx(2.0) and ent["calibration"]["write_factor"] == 1.0
    # intra: FETCH medians of {100, 300, 200} KiB = 200 KiB -> 400 KiB; WRITE median 8 KiB
    assert ent["intra"]["fetch_kib"] == 200 and ent["intra"]["write_kib"] == 8
    assert ent["intra"]["bytes_per_launch"] == pytest.approx(200 * 1024 * 2 + 8 * 1024)
    assert ent["intra"]["rocprof_avg_us"] == pytest.approx(101.5)
    assert bench.traffic_for("wl", ["intra", "scan_full"]) == pytest.approx(
        (200 * 2 + 8) * 1024 + (10 * 2 + 4) * 1024)
    # a figure taken on other source code is dropped
    monkeypatch.setattr(bench, "source_sha", lambda k: "0" * 16)
    assert bench.traffic_for("wl", ["intra"]) is None
