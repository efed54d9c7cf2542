"""Parity of the forward's options against the fp64 oracle: raw-logit beta with the
in-kernel sigmoid, bf16 state input/output, and the per-chunk states hc (the
FlashKDA page's input/state variants; per-chunk states as kept for the chunked
backward).  Same tolerance as the main parity tests:
    max|x - x_ref| / max|x_ref| <= 1e-2 for o, ht and hc.
"""
import numpy as np
import pytest

from oracle import chunked, recurrent
from synth.inputs import make_inputs, round_to_bf16

from _gpu_util import FIELDS, nerr, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


def run(d, t, **kw):
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    out = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"],
                  cu_seqlens=t["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return [None if x is None else x.float().cpu().numpy().astype(np.float64) for x in out]


def test_beta_logits_sigmoid_in_kernel():
    import torch
    d = make_inputs(71, B=1, T=64 * 3 + 17, HQK=1, HV=2, K=128, V=64, has_h0=True)
    rng = np.random.default_rng(710)
    x = round_to_bf16(3.0 * rng.standard_normal(d["beta"].shape))
    x[0, :6, 0] = [40.0, -40.0, 12.0, -12.0, 0.0, 88.0]     # saturating logits (bf16-exact)
    t = to_device(d)
    t["beta"] = torch.from_numpy(x).to(torch.bfloat16).cuda()
    o, ht = run(d, t, beta_logits=True)
    ref = dict(d, beta=1.0 / (1.0 + np.exp(-x)))
    o_ref, ht_ref = recurrent(**{k: ref[k] for k in FIELDS}, scale=d["scale"], h0=d["h0"])
    eo, eh = nerr(o, o_ref), nerr(ht, ht_ref)
    print(f"  o err {eo:.3e}  ht err {eh:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and eo <= TOL and eh <= TOL


def test_bf16_state_in_and_out():
    import torch
    d = make_inputs(72, B=2, T=150, HQK=2, HV=4, K=64, V=48, has_h0=True)
    h0_bf = round_to_bf16(d["h0"])
    t = to_device(d)
    t["h0"] = torch.from_numpy(h0_bf).to(torch.bfloat16).cuda()
    o, ht = run(d, t, state_dtype=torch.bfloat16)
    o_ref, ht_ref = recurrent(**{k: d[k] for k in FIELDS}, scale=d["scale"], h0=h0_bf)
    eo, eh = nerr(o, o_ref), nerr(ht, ht_ref)
    print(f"  o err {eo:.3e}  ht err {eh:.3e}", flush=True)
    assert eo <= TOL and eh <= TOL
    # ht is the bf16 rounding of an fp32 state: every value is bf16-exact
    assert np.array_equal(ht, round_to_bf16(ht))


@pytest.mark.parametrize("case", ["fixed", "varlen", "varlen_bf16"])
def test_chunk_states(case):
    import torch
    if case == "fixed":
        d = make_inputs(73, B=2, T=200, HQK=1, HV=2, K=64, V=32, has_h0=True)
    else:
        d = make_inputs(74, B=1, T=0, HQK=2, HV=4, K=128, V=64, has_h0=True, lengths=[70, 0, 129, 1, 64])
    t = to_device(d)
    sdt = torch.bfloat16 if case == "varlen_bf16" else torch.float32
    h0_used = d["h0"]
    if sdt == torch.bfloat16:
        h0_used = round_to_bf16(d["h0"])
        t["h0"] = torch.from_numpy(h0_used).to(torch.bfloat16).cuda()
    # hc starts as zeros: the rows past the written chunks must stay untouched
    from gated_delta_rule_chunked_amd import max_chunks
    N = d["B"] if d["cu_seqlens"] is None else len(d["cu_seqlens"]) - 1
    C = max_chunks(d["T"], N, d["B"], d["cu_seqlens"] is not None)
    hc0 = torch.zeros((C, d["HV"], d["K"], d["V"]), dtype=sdt, device="cuda")
    o, ht, hc = run(d, t, output_chunk_states=True, state_dtype=sdt, hc=hc0)
    o_plain, ht_plain = run(d, t, state_dtype=sdt)
    assert np.array_equal(o, o_plain) and np.array_equal(ht, ht_plain)   # hc changes nothing else
    _, _, inter = chunked(**{k: d[k] for k in FIELDS}, scale=d["scale"], h0=h0_used,
                          cu_seqlens=d["cu_seqlens"], chunk=64, return_intermediates=True)
    # varlen: hc has room for ceil(T/64) + N chunks; the first sum ceil(len/64) are written
    assert hc.shape[0] == (len(inter) if case == "fixed" else (d["T"] + 63) // 64 + len(d["cu_seqlens"]) - 1)
    assert np.all(hc[len(inter):] == 0)
    hc = hc[:len(inter)]
    ref = np.stack([ci["h"] for ci in inter])
    e = nerr(hc, ref)
    print(f"  hc err {e:.3e} over {len(inter)} chunks", flush=True)
    assert np.all(np.isfinite(hc)) and e <= TOL
