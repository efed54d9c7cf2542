"""Chunk length 16 (FlashKDA's recurrence kernel uses CHUNK = 16): the state is
updated every 16 tokens and the intra-chunk terms span 16 tokens.  o and ht are
the same quantities as at chunk 64, so every case is compared element by element
with the token recurrence at the stated bar (max|x - x_ref| / max|x_ref| <= 1e-2),
outputs starting as NaN; the same inputs at chunk 64 differ only by rounding."""
import numpy as np
import pytest

from synth import make_config_inputs
from synth.inputs import make_inputs
from oracle import recurrent

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


def run16(d, chunk=16, seg_chunks=0, t=None):
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    t = to_device(d) if t is None else t
    N = d["B"] if d["cu_seqlens"] is None else len(d["cu_seqlens"]) - 1
    o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ht = torch.full((N, d["HV"], d["K"], d["V"]), float("nan"), dtype=torch.float32, device="cuda")
    kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"], cu_seqlens=t["cu_seqlens"],
            o=o, ht=ht, chunk=chunk, seg_chunks=seg_chunks)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), ht.cpu().numpy().astype(np.float64)


def reference(d):
    return recurrent(**{k: d[k] for k in FIELDS}, scale=d["scale"], h0=d["h0"], cu_seqlens=d["cu_seqlens"])


def check(d, got, tol=TOL, what=""):
    o, ht = got
    o_ref, ht_ref = reference(d)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    eo, eh = nerr(o, o_ref), nerr(ht, ht_ref)
    print(f"  {what}: o err {eo:.3e}  ht err {eh:.3e}", flush=True)
    assert eo <= tol and eh <= tol


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 200, 257])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 48), (128, 16)])
def test_chunk16_ragged_lengths(T, K, V):
    d = make_inputs(300 + T, B=2, T=T, HQK=1, HV=2, K=K, V=V, has_h0=True)
    check(d, run16(d), what=f"T={T} K={K} V={V}")


def test_chunk16_varlen_grouped_heads_with_empty_and_tiny_sequences():
    d = make_inputs(311, B=1, T=0, HQK=2, HV=4, K=128, V=64, has_h0=True,
                    lengths=[0, 1, 15, 16, 17, 64, 130, 0, 7, 300])
    o, ht = run16(d)
    check(d, (o, ht), what="varlen")
    assert np.array_equal(ht[0], d["h0"][0].astype(np.float64))   # empty sequences keep h0
    assert np.array_equal(ht[7], d["h0"][7].astype(np.float64))


@pytest.mark.parametrize("seg", [1, 2, 3])
def test_chunk16_forced_segments(seg):
    # the state pass's b and M and the full pass's prologue, four 16-row updates per record
    d = make_inputs(321, B=2, T=64 * 7 + 23, HQK=1, HV=2, K=128, V=80, has_h0=True)
    check(d, run16(d, seg_chunks=seg), what=f"segments of {seg}")
    dv = make_inputs(322, B=1, T=0, HQK=1, HV=2, K=64, V=32, has_h0=True, lengths=[257, 0, 130, 64, 5])
    check(dv, run16(dv, seg_chunks=seg), what=f"varlen, segments of {seg}")


def test_chunk16_gates_far_below_the_floor():
    d = make_inputs(331, B=1, T=200, HQK=1, HV=2, K=128, V=64, has_h0=True)
    g = d["g"]
    g[0, 16:32, 0, :] = -np.inf          # a whole 16-row chunk
    g[0, 40:56, 1, ::3] = -30.0
    g[0, 199, :, :] = -np.inf
    check(d, run16(d), what="floored gates")


def test_chunk16_and_chunk64_differ_only_by_rounding():
    d = make_inputs(341, B=1, T=64 * 5 + 9, HQK=2, HV=4, K=128, V=64, has_h0=True)
    t = to_device(d)
    o16, h16 = run16(d, t=t)
    o64, h64 = run16(d, chunk=64, t=t)
    assert nerr(o16, o64) <= 5e-3 and nerr(h16, h64) <= 5e-3


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_chunk16_workloads(cfg):
    # the benchmarked 8192-token, 32-head workload included (every head compared)
    d = make_config_inputs(cfg)
    check(d, run16(d), what=f"workload {cfg}")
