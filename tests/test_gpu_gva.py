"""Grouped value heads (GVA) at group sizes other than two, through the C ABI.

Value head h reads q/k head h / (HV / HQK); beta and g are per value head.  Every
case runs with o and ht pre-filled with NaN and is compared element by element with
the token recurrence (the same bar as the other parity tests), on the library's own
scan choice, on forced segments of the 64-column scan and at chunk 16; a grouped run
must also equal the run with q and k repeated per value head, bit for bit.
"""
import numpy as np
import pytest

from synth.inputs import make_inputs
from oracle import recurrent

from _gpu_util import FIELDS, nerr, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-2
GROUPS = [(1, 4), (2, 8), (1, 8), (3, 12), (1, 5)]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


def run(d, **kw):
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    t = to_device(d)
    N = t["q"].shape[0] if t["cu_seqlens"] is None else t["cu_seqlens"].numel() - 1
    o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device=t["v"].device)
    ht = torch.full((N, t["v"].shape[2], t["q"].shape[3], t["v"].shape[3]), float("nan"),
                    dtype=torch.float32, device=t["v"].device)
    kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"],
            cu_seqlens=t["cu_seqlens"], o=o, ht=ht, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), ht.cpu().numpy().astype(np.float64)


def check(d, o, ht):
    o_ref, ht_ref = recurrent(**{k: d[k] for k in FIELDS}, scale=d["scale"], h0=d["h0"],
                              cu_seqlens=d["cu_seqlens"])
    eo, eh = nerr(o, o_ref), nerr(ht, ht_ref)
    print(f"  o err {eo:.3e}  ht err {eh:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    assert eo <= TOL and eh <= TOL


@pytest.mark.parametrize("opts", [{}, {"seg_chunks": 2}, {"chunk": 16}], ids=["plan", "seg2", "chunk16"])
@pytest.mark.parametrize("HQK,HV", GROUPS)
def test_group_sizes_fixed_length(HQK, HV, opts):
    d = make_inputs(400 + 10 * HQK + HV, B=2, T=64 * 3 + 29, HQK=HQK, HV=HV, K=128, V=64, has_h0=True)
    check(d, *run(d, **opts))


@pytest.mark.parametrize("opts", [{}, {"seg_chunks": 1}, {"chunk": 16}], ids=["plan", "seg1", "chunk16"])
@pytest.mark.parametrize("HQK,HV", [(1, 4), (2, 8), (3, 12)])
def test_group_sizes_varlen(HQK, HV, opts):
    d = make_inputs(500 + 10 * HQK + HV, B=1, T=0, HQK=HQK, HV=HV, K=128, V=32, has_h0=True,
                    lengths=[130, 0, 64, 257, 3])
    check(d, *run(d, **opts))


@pytest.mark.parametrize("opts", [{}, {"seg_chunks": 2}], ids=["plan", "seg2"])
def test_group_of_four_equals_repeated_heads_bitwise(opts):
    d = make_inputs(601, B=1, T=64 * 4 + 9, HQK=2, HV=8, K=64, V=48, has_h0=True)
    o1, h1 = run(d, **opts)
    rep = dict(d, q=np.repeat(d["q"], 4, axis=2), k=np.repeat(d["k"], 4, axis=2), HQK=8)
    o2, h2 = run(rep, **opts)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
    check(d, o1, h1)
