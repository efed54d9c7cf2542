"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerance (the stated bar for bf16 I/O with fp32 accumulation):
    max|o - o_ref| / max|o_ref| <= 1e-2   and   max|ht - ht_ref| / max|ht_ref| <= 1e-2
on the same seeded bf16 inputs.  Every case, the full-size workloads in the exact
launch configuration the benchmark times included, compares every element of o
and ht against the token recurrence; outputs start as NaN so that an element the
kernels never write fails.
"""
import numpy as np
import pytest

from synth import make_config_inputs
from synth.inputs import make_inputs
from oracle import chunked, recurrent

from _gpu_util import FIELDS, nerr, run_hip, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


def full_oracle(d):
    a = {k: d[k] for k in FIELDS}
    return recurrent(**a, scale=d["scale"], h0=d["h0"], cu_seqlens=d["cu_seqlens"])


def check(o, ht, o_ref, ht_ref, tol=TOL):
    eo = nerr(o, o_ref)
    eh = nerr(ht, ht_ref) if ht_ref is not None else 0.0
    print(f"  o err {eo:.3e}  ht err {eh:.3e}", flush=True)
    assert np.all(np.isfinite(o))
    assert eo <= tol and eh <= tol


# -------------------------------------------------------------- workloads


@pytest.mark.parametrize("cfg", [1, 2])
def test_small_workloads_full(cfg):
    d = make_config_inputs(cfg)
    o, ht = run_hip(d)
    o_ref, ht_ref = full_oracle(d)
    check(o, ht, o_ref, ht_ref)


@pytest.mark.parametrize("cfg", [3, 5])
def test_large_workloads_every_head(cfg):
    # the launch configuration the benchmark times (library's own scan choice); o and ht
    # start as NaN and every element of every head is compared with the token recurrence
    d = make_config_inputs(cfg)
    o, ht = run_hip(d)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    o_ref, ht_ref = full_oracle(d)
    for hv in range(d["HV"]):
        eo, eh = nerr(o[:, :, hv], o_ref[:, :, hv]), nerr(ht[:, hv], ht_ref[:, hv])
        assert eo <= TOL and eh <= TOL, (hv, eo, eh)
    print(f"  all {d['HV']} heads:", end="")
    check(o, ht, o_ref, ht_ref)


def test_varlen_workload_every_sequence_and_head():
    d = make_config_inputs(4)
    o, ht = run_hip(d)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    o_ref, ht_ref = full_oracle(d)
    cu = d["cu_seqlens"]
    worst = 0.0
    for seq in range(len(cu) - 1):
        for hv in range(d["HV"]):
            rows = slice(int(cu[seq]), int(cu[seq + 1]))
            eo = nerr(o[0, rows, hv], o_ref[0, rows, hv])
            eh = nerr(ht[seq, hv], ht_ref[seq, hv])
            worst = max(worst, eo, eh)
            assert eo <= TOL and eh <= TOL, (seq, hv, eo, eh)
    print(f"  {len(cu) - 1} sequences x {d['HV']} heads, worst {worst:.3e}:", end="")
    check(o, ht, o_ref, ht_ref)


# ----------------------------------------------------------- edge cases


@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 200, 257])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 48), (128, 256), (64, 16)])
def test_ragged_lengths(T, K, V):
    d = make_inputs(100 + T, B=2, T=T, HQK=1, HV=2, K=K, V=V, has_h0=True)
    o, ht = run_hip(d)
    check(o, ht, *full_oracle(d))


def test_varlen_with_empty_and_tiny_sequences_gva():
    d = make_inputs(31, B=1, T=0, HQK=2, HV=4, K=128, V=32, has_h0=True,
                    lengths=[0, 1, 64, 65, 130, 0, 7, 300])
    o, ht = run_hip(d)
    check(o, ht, *full_oracle(d))
    assert np.array_equal(ht[0], d["h0"][0].astype(np.float64))
    assert np.array_equal(ht[5], d["h0"][5].astype(np.float64))


def test_many_chunks_no_initial_state_k64():
    # NT >= 4 (long serial chain), h0 = None, no final state requested
    d = make_inputs(41, B=1, T=64 * 9 + 5, HQK=1, HV=1, K=64, V=64, has_h0=False)
    o, ht = run_hip(d, output_final_state=False)
    assert ht is None
    o_ref, _ = full_oracle(d)
    check(o, None, o_ref, None)


def test_strong_decay_stays_finite():
    # per-token gates near -8 (decay ~3e-4 per token): factors up to e^64, still exact
    d = make_inputs(42, B=1, T=192, HQK=1, HV=2, K=128, V=64, has_h0=True, g_mean=-8.0)
    assert d["g"].min() < -9
    o, ht = run_hip(d)
    check(o, ht, *full_oracle(d))


def test_gates_below_the_supported_range():
    # gates below -10 (here -30, -1000 and -inf on whole tokens and on single
    # dimensions) are raised to -10 in the intra stage; the outputs stay finite and
    # within the tolerance of the exact recurrence, which decays those tokens fully
    d = make_inputs(43, B=1, T=200, HQK=1, HV=2, K=128, V=64, has_h0=True)
    g = d["g"]
    g[0, 5, 0, :] = -30.0
    g[0, 63, 1, :] = -1000.0
    g[0, 64, 0, :] = -np.inf
    g[0, 70:90, 1, 3] = -np.inf
    g[0, 100:140:7, :, 17] = -30.0
    g[0, 199, :, :] = -np.inf
    o, ht = run_hip(d)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    check(o, ht, *full_oracle(d))


@pytest.mark.parametrize("K", [128, 64])
def test_whole_blocks_at_and_below_the_gate_floor(K):
    """Whole 16-token blocks of gates at or below the floor (-11, -30, -inf; every
    dimension or some), among them a chunk's last block and the last block of the
    final, ragged chunk, and a pair of neighbouring blocks whose decay sits inside
    them while their facing tokens stay close (the case where the cross-block gate
    factor of the 16-row blocks would underflow in fp32 if it were referenced to
    the block midpoints).  o and ht are compared with the exact token recurrence."""
    T = 64 * 3 + 40
    d = make_inputs(44, B=1, T=T, HQK=1, HV=2, K=K, V=64, has_h0=True)
    g = d["g"]
    g[0, 48:64, 0, :] = -11.0            # chunk 0's last block, every dimension
    g[0, 48:64, 1, :] = -np.inf
    g[0, 64:96, 0, : K // 3] = -30.0     # two blocks, some dimensions
    g[0, 64:96, 1, K // 2:] = -np.inf
    # chunk 2: decay inside block 1 (rows 144..158) and block 2 (rows 161..175),
    # tokens 159 and 160 between them ungated
    g[0, 144:159, 0, :] = -30.0
    g[0, 161:176, 0, :] = -30.0
    g[0, 144:159, 1, ::2] = -np.inf
    g[0, 161:176, 1, ::2] = -np.inf
    g[0, 159:161, :, :] = 0.0
    g[0, 208:T, 0, :] = -11.0            # the final chunk's last full block and its tail
    g[0, 208:T, 1, :] = -np.inf
    t = to_device(d)
    import torch
    o_buf = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    o, ht = run_hip(d, dev=t, o=o_buf)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    check(o, ht, *full_oracle(d))


def test_intermediates_match_chunked_oracle():
    """The intra stage alone: qg, w, kg, Aqk, Tm diag(beta), exp(G) against the
    chunked oracle's per-chunk intermediates."""
    import torch
    from gated_delta_rule_chunked_amd import (alloc_workspace, kda_debug_unpack, kda_fwd_intra,
                                              make_args)
    d = make_inputs(51, B=1, T=150, HQK=1, HV=2, K=128, V=64, has_h0=False)
    t = to_device(d)
    B, T, HV, K = 1, 150, 2, 128
    a = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"])
    wsp = alloc_workspace(a, "cuda")
    a.workspace, a.workspace_bytes = wsp.data_ptr(), wsp.numel()
    kda_fwd_intra(a)
    outs = {n: torch.full((B, T, HV, K), float("nan"), dtype=torch.bfloat16, device="cuda")
            for n in ("qg", "w", "kg")}
    outs["aqk"] = torch.full((B, T, HV, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    outs["tmb"] = torch.full((B, T, HV, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    outs["alpha"] = torch.full((B, T, HV, K), float("nan"), dtype=torch.float32, device="cuda")
    kda_debug_unpack(a, **outs)
    torch.cuda.synchronize()
    got = {n: x.float().cpu().numpy().astype(np.float64)[0] for n, x in outs.items()}
    _, _, inter = chunked(**{k: d[k] for k in FIELDS}, scale=d["scale"], chunk=64,
                          return_intermediates=True)
    for ci in inter:
        r0, L = ci["row0"], ci["rows"]
        rows = slice(r0, r0 + L)
        ref = {
            "qg": d["scale"] * ci["qg"], "w": ci["w"], "kg": ci["kg"],
            "aqk": np.transpose(ci["Aqk"], (1, 0, 2)),                      # [i, h, j]
            "tmb": np.transpose(ci["Tm"] * np.asarray(d["beta"][0, rows]).T[:, None, :], (1, 0, 2)),
            "alpha": np.broadcast_to(np.exp(ci["gd"])[None], (L, HV, K)),
        }
        for n, rv in ref.items():
            gv = got[n][rows]
            if n in ("aqk", "tmb"):
                gv = gv[:, :, :L]
            e = nerr(gv, rv)
            print(f"  chunk@{r0} {n}: {e:.2e}", flush=True)
            assert np.all(np.isfinite(gv)) and e <= TOL, (n, r0, e)
        if L < 64:   # columns past the chunk's rows are exact zeros
            assert np.all(got["aqk"][rows][:, :, L:] == 0) and np.all(got["tmb"][rows][:, :, L:] == 0)


# ------------------------------------------------ hazards and invariants


def test_poisoned_workspace_and_output_are_fully_overwritten():
    import torch
    d = make_inputs(61, B=1, T=64 * 5 + 3, HQK=1, HV=2, K=128, V=32, has_h0=True)
    t = to_device(d)
    o_clean, ht_clean = run_hip(d, dev=t)
    from gated_delta_rule_chunked_amd import alloc_workspace, make_args
    ws = alloc_workspace(make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], t["h0"]), "cuda")
    ws.fill_(0xFF)                                             # NaN in every fp32/bf16 view
    o_buf = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    o, ht = run_hip(d, dev=t, workspace=ws, o=o_buf)
    assert np.all(np.isfinite(o)) and np.array_equal(o, o_clean) and np.array_equal(ht, ht_clean)


def test_back_to_back_calls_into_separate_buffers():
    d1 = make_inputs(71, B=1, T=300, HQK=2, HV=2, K=128, V=64, has_h0=True)
    d2 = make_inputs(72, B=1, T=300, HQK=2, HV=2, K=128, V=64, has_h0=True)
    t1, t2 = to_device(d1), to_device(d2)
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    r1 = kda_fwd(*(t1[k] for k in FIELDS), scale=d1["scale"], h0=t1["h0"])
    r2 = kda_fwd(*(t2[k] for k in FIELDS), scale=d2["scale"], h0=t2["h0"])
    torch.cuda.synchronize()
    s1, s2 = run_hip(d1, dev=t1), run_hip(d2, dev=t2)
    assert np.array_equal(r1[0].float().cpu().numpy(), s1[0]) and np.array_equal(r1[1].cpu().numpy(), s1[1])
    assert np.array_equal(r2[0].float().cpu().numpy(), s2[0]) and np.array_equal(r2[1].cpu().numpy(), s2[1])


def test_causality_bitwise_at_block_boundary():
    d = make_inputs(81, B=1, T=256, HQK=1, HV=2, K=128, V=32, has_h0=True)
    o1, _ = run_hip(d)
    e = dict(d)
    rng = np.random.default_rng(5)
    for k in ("q", "k", "v"):
        e[k] = d[k].copy()
        e[k][0, 80:] = np.float32(0.5) * np.sign(rng.standard_normal(e[k][0, 80:].shape)).astype(np.float32)
    e["g"] = d["g"].copy()
    e["g"][0, 80:] = -1.0
    e["beta"] = d["beta"].copy()
    e["beta"][0, 80:] = 0.75
    o2, _ = run_hip(e)
    # rows before the first perturbed 16-row block are bit-identical
    assert np.array_equal(o1[0, :80], o2[0, :80])
    assert not np.allclose(o1[0, 80:], o2[0, 80:])


def test_split_resume():
    import torch
    d = make_inputs(91, B=1, T=400, HQK=1, HV=2, K=128, V=64, has_h0=True)
    o, ht = run_hip(d)
    first = dict(d, **{k: d[k][:, :192] for k in FIELDS}, T=192)
    second = dict(d, **{k: d[k][:, 192:] for k in FIELDS}, T=208)
    oa, ha = run_hip(first)
    second["h0"] = ha.astype(np.float32)
    ob, hb = run_hip(second)
    assert nerr(np.concatenate([oa, ob], axis=1), o) <= 2e-3 and nerr(hb, ht) <= 2e-3


def test_grouped_heads_equal_repeated_heads_bitwise():
    d = make_inputs(101, B=1, T=260, HQK=2, HV=4, K=128, V=32, has_h0=True)
    o1, h1 = run_hip(d)
    rep = dict(d, q=np.repeat(d["q"], 2, axis=2), k=np.repeat(d["k"], 2, axis=2), HQK=4)
    o2, h2 = run_hip(rep)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


def test_varlen_equals_separate_runs_bitwise():
    lengths = [70, 0, 129, 1]
    d = make_inputs(111, B=1, T=0, HQK=1, HV=2, K=128, V=32, has_h0=True, lengths=lengths)
    o, ht = run_hip(d)
    cu = d["cu_seqlens"]
    for n in range(len(lengths)):
        if lengths[n] == 0:
            continue
        part = dict(d, **{k: d[k][:, cu[n]:cu[n + 1]] for k in FIELDS}, T=lengths[n],
                    h0=d["h0"][n:n + 1], cu_seqlens=None, N=1)
        on, hn = run_hip(part)
        assert np.array_equal(o[:, cu[n]:cu[n + 1]], on) and np.array_equal(ht[n], hn[0])


def test_rejected_cu_seqlens_poisons_outputs():
    import torch
    d = make_inputs(121, B=1, T=0, HQK=1, HV=1, K=64, V=16, has_h0=False, lengths=[100, 50, 50])
    d["cu_seqlens"] = np.array([0, 100, 50, 200], dtype=np.int64)   # not non-decreasing
    o, ht = run_hip(d)
    assert np.all(np.isnan(o)) and np.all(np.isnan(ht))


def test_varlen_serial_scan_longest_first_order():
    # 40 short sequences x 3 heads: the 16-column serial scan, its (sequence, head)
    # units handed out longest first (120 units, not a multiple of the eight XCDs);
    # every o row is checked, starting from NaN
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd, kda_fwd_scan_plan, make_args
    rng = np.random.default_rng(146)
    lengths = [int(x) for x in rng.integers(0, 200, size=40)]
    lengths[7] = 0
    d = make_inputs(147, B=1, T=0, HQK=3, HV=3, K=128, V=128, has_h0=True, lengths=lengths)
    t = to_device(d)
    o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    a = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], t["h0"], t["cu_seqlens"], o, None)
    assert kda_fwd_scan_plan(a) == 0   # the serial scan
    out = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"],
                  cu_seqlens=t["cu_seqlens"], o=o)
    torch.cuda.synchronize()
    o_np, ht_np = [x.float().cpu().numpy().astype(np.float64) for x in out]
    assert np.all(np.isfinite(o_np))
    check(o_np, ht_np, *full_oracle(d))
    assert np.array_equal(ht_np[7], d["h0"][7].astype(np.float64))
