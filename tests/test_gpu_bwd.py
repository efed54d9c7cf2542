"""Parity of the backward reverse state scan (kda_bwd_dhu) against the fp64 oracle.

The scan's inputs are the forward's chunk operands, computed by the oracle
(``stage_inputs``) and rounded to the kernel's input dtypes; the oracle's
``bwd_dhu`` then runs on exactly those rounded values.  Bar, as for the forward:
    max|x - x_ref| / max|x_ref| <= 1e-2   for dv2, dhc and dh0.
"""
import math

import numpy as np
import pytest

from oracle import bwd_dhu, stage_inputs
from synth.inputs import make_grads, make_inputs, round_to_bf16

from _gpu_util import FIELDS, nerr

pytestmark = pytest.mark.gpu
TOL = 1e-2
LN2 = math.log(2.0)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


def scan_inputs(d, gr, heads=None, zero_dv=False):
    """The scan's inputs in the kernel's dtypes (float64 arrays holding bf16 / fp32
    values).  ``heads``: restrict to these value heads (with their q/k heads)."""
    a = {k: d[k] for k in FIELDS}
    do = gr["do"]
    dht = gr["dht"]
    if heads is not None:
        hq = [h // (d["HV"] // d["HQK"]) for h in heads]
        a = dict(q=a["q"][:, :, hq], k=a["k"][:, :, hq], v=a["v"][:, :, heads], g=a["g"][:, :, heads],
                 beta=a["beta"][:, :, heads])
        do = do[:, :, heads]
        dht = None if dht is None else dht[:, heads]
    si = stage_inputs(**a, scale=d["scale"], do=do, cu_seqlens=d["cu_seqlens"])
    x = {n: round_to_bf16(si[n]) for n in ("qg", "kg", "w")}
    x["g2"] = (si["gcum"] / LN2).astype(np.float32)
    x["dv"] = None if zero_dv else round_to_bf16(si["dv_in"])
    x["do"] = np.asarray(do, dtype=np.float64)
    x["dht"] = dht
    return x


def reference(x, d):
    gcum = x["g2"].astype(np.float64) * LN2     # the kernel's exp2(g2) is exp(gcum)
    dv = np.zeros_like(x["do"]) if x["dv"] is None else x["dv"]
    return bwd_dhu(x["qg"], x["kg"], x["w"], gcum, x["do"], dv, d["scale"], dht=x["dht"],
                   cu_seqlens=d["cu_seqlens"])


def run_gpu(x, d, state_dtype=None, checkpoint_dtype=None, **kw):
    import torch
    from gated_delta_rule_chunked_amd import kda_bwd_dhu

    def dev(a, dt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    bf = torch.bfloat16
    sdt = torch.float32 if state_dtype is None else state_dtype
    cu = None if d["cu_seqlens"] is None else torch.from_numpy(np.asarray(d["cu_seqlens"], np.int64)).cuda()
    out = kda_bwd_dhu(dev(x["qg"], bf), dev(x["kg"], bf), dev(x["w"], bf), dev(x["g2"], torch.float32),
                      dev(x["do"], bf), dev(x["dv"], bf), dev(x["dht"], sdt), scale=d["scale"], cu_seqlens=cu,
                      state_dtype=state_dtype, checkpoint_dtype=checkpoint_dtype, **kw)
    torch.cuda.synchronize()
    res = [None if t is None else t.float().cpu().numpy().astype(np.float64) for t in out]
    if res[1] is not None and d["cu_seqlens"] is not None:   # varlen: rows past the chunk total unwritten
        cu = np.asarray(d["cu_seqlens"])
        res[1] = res[1][:int(sum((cu[i + 1] - cu[i] + 63) // 64 for i in range(len(cu) - 1)))]
    return res


def check(got, ref, what=""):
    errs = []
    for name, a, b in zip(("dv2", "dhc", "dh0"), got, ref):
        if a is None:
            continue
        assert a.shape == b.shape, (name, a.shape, b.shape)
        assert np.all(np.isfinite(a)), name
        e = nerr(a, b)
        errs.append(f"{name} {e:.2e}")
        assert e <= TOL, (what, name, e)
    print(f"  {what}: " + "  ".join(errs), flush=True)


@pytest.mark.parametrize("B,T,HQK,HV,K,V", [
    (2, 64 * 3 + 17, 1, 2, 128, 64),     # ragged tail, four value tiles
    (1, 256, 1, 1, 64, 64),              # K = 64
    (1, 64, 2, 4, 128, 16),              # one chunk, grouped heads, one value tile
    (1, 5, 1, 1, 128, 32),               # a single partial chunk
])
def test_bwd_dhu_fixed_length(B, T, HQK, HV, K, V):
    d = make_inputs(81, B=B, T=T, HQK=HQK, HV=HV, K=K, V=V, has_h0=False)
    gr = make_grads(d, 810)
    x = scan_inputs(d, gr)
    check(run_gpu(x, d), reference(x, d), f"B{B} T{T} HV{HV} K{K} V{V}")


def test_bwd_dhu_varlen_with_empty_and_ragged_sequences():
    d = make_inputs(82, B=1, T=0, HQK=1, HV=2, K=128, V=32, has_h0=True, lengths=[100, 0, 64, 1, 300, 0])
    gr = make_grads(d, 820)
    x = scan_inputs(d, gr)
    got, ref = run_gpu(x, d), reference(x, d)
    check(got, ref, "varlen")
    # empty sequences: dh0 = dht exactly
    for n in (1, 5):
        assert np.array_equal(got[2][n], gr["dht"][n].astype(np.float64))


def test_bwd_dhu_bf16_checkpoints_and_state():
    import torch
    d = make_inputs(83, B=2, T=200, HQK=2, HV=2, K=64, V=48, has_h0=False)
    gr = make_grads(d, 830)
    gr["dht"] = round_to_bf16(gr["dht"])
    x = scan_inputs(d, gr)
    ref = reference(x, d)
    got = run_gpu(x, d, state_dtype=torch.bfloat16, checkpoint_dtype=torch.bfloat16)
    check(got, ref, "bf16 dhc + bf16 dht/dh0")
    # the bf16 checkpoint is the fp32 one rounded to nearest even
    got32 = run_gpu(x, d)
    assert np.array_equal(got[1], round_to_bf16(got32[1]))
    assert np.array_equal(got[0], got32[0])          # dv2 does not depend on the checkpoint dtype


def test_bwd_dhu_zero_dv_no_dht_and_skipped_outputs():
    d = make_inputs(84, B=1, T=64 * 5, HQK=1, HV=1, K=128, V=32, has_h0=False)
    gr = make_grads(d, 840, has_dht=False)
    x = scan_inputs(d, gr, zero_dv=True)
    ref = reference(x, d)
    check(run_gpu(x, d), ref, "dv = 0, dht = 0")
    dv2, dhc, dh0 = run_gpu(x, d, output_dh0=False, output_checkpoints=False)
    assert dhc is None and dh0 is None
    assert nerr(dv2, ref[0]) <= TOL


def test_bwd_dhu_small_batched_workload():
    # the B=2, T=2048, four-head, K=V=128 shape
    d = make_inputs(2, B=2, T=2048, HQK=4, HV=4, K=128, V=128, has_h0=True)
    gr = make_grads(d, 20)
    x = scan_inputs(d, gr)
    check(run_gpu(x, d, checkpoint_dtype=None), reference(x, d), "B2 T2048 H4")


def test_bwd_dhu_prefill_size_all_heads():
    # The 8192-token, 32-head, K=V=128 prefill shape in the launch the benchmark
    # times (bf16 checkpoints).  Heads are independent, so three seeded heads are
    # tiled over the 32 (head h carries head h % 3) and every head is checked
    # against the oracle of its source head.
    import torch
    d3 = make_inputs(3, B=1, T=8192, HQK=3, HV=3, K=128, V=128, has_h0=False)
    gr = make_grads(d3, 30)
    x3 = scan_inputs(d3, gr)
    ref = reference(x3, d3)
    src = [h % 3 for h in range(32)]
    x = {k: (None if v is None else (v[:, src] if k == "dht" else v[:, :, src])) for k, v in x3.items()}
    d = dict(d3, HV=32, HQK=32)
    dv2, dhc, dh0 = run_gpu(x, d, checkpoint_dtype=torch.bfloat16)
    tiled = [ref[0][:, :, src], ref[1][:, src], ref[2][:, src]]
    check([dv2, dhc, dh0], tiled, "prefill T8192 H32")
