"""kda_fwd_no_alloc: the forward on the library's static per-device scratch, for
callers that cannot allocate.  Called through the C ABI; its outputs must equal
those of kda_fwd with a caller workspace (the same kernels), call after call on the
shared buffer, and meet the oracle's tolerance."""
import ctypes

import numpy as np
import pytest

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


def run_both(d):
    import torch
    from gated_delta_rule_chunked_amd import alloc_workspace, kda_fwd_raw, load_library, make_args
    from gated_delta_rule_chunked_amd.kda import KDA_OK
    t = to_device(d)
    N = d["B"] if d["cu_seqlens"] is None else len(d["cu_seqlens"]) - 1
    outs = []
    for no_alloc in (False, True):
        o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        ht = torch.full((N, d["HV"], d["K"], d["V"]), float("nan"), dtype=torch.float32, device="cuda")
        a = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], t["h0"], t["cu_seqlens"], o, ht)
        if no_alloc:
            a.workspace, a.workspace_bytes = None, 0   # ignored by the entry point
            st = load_library().kda_fwd_no_alloc(ctypes.byref(a))
            assert st == KDA_OK, st
        else:
            ws = alloc_workspace(a, "cuda")
            a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
            kda_fwd_raw(a)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy().astype(np.float64), ht.cpu().numpy().astype(np.float64)))
    return outs


def test_no_alloc_matches_the_workspace_entry_on_consecutive_calls():
    # a large call (4,096 tokens, two heads: the segmented scan, with its segment end
    # states and transitions in the scratch), then a smaller one (fixed length, K = 64),
    # then varlen with grouped heads and empty / one-token sequences (the serial scan)
    d1 = make_inputs(203, B=1, T=4096, HQK=1, HV=2, K=128, V=128, has_h0=True)
    d2 = make_inputs(202, B=2, T=150, HQK=1, HV=2, K=64, V=32, has_h0=False)
    d3 = make_inputs(201, B=1, T=0, HQK=2, HV=4, K=128, V=128, has_h0=True, lengths=[1500, 70, 0, 2100, 1])
    for d in (d1, d2, d3):
        (o_ws, ht_ws), (o_na, ht_na) = run_both(d)
        assert np.all(np.isfinite(o_na)) and np.all(np.isfinite(ht_na))
        assert np.array_equal(o_na, o_ws) and np.array_equal(ht_na, ht_ws)
        o_ref, ht_ref = recurrent(**{k: d[k] for k in FIELDS}, scale=d["scale"], h0=d["h0"],
                                  cu_seqlens=d["cu_seqlens"])
        eo, eh = nerr(o_na, o_ref), nerr(ht_na, ht_ref)
        print(f"  T={d['T']} HV={d['HV']} K={d['K']}: o err {eo:.2e} ht err {eh:.2e}", flush=True)
        assert eo <= TOL and eh <= TOL


def test_no_alloc_rejects_shapes_beyond_its_buffer():
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd_workspace_bytes, load_library, make_args
    from gated_delta_rule_chunked_amd.kda import KDA_ERR_TOO_LARGE, KDA_NO_ALLOC_MAX_BYTES
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")  # noqa: E731
    q = z(1, 8192, 32, 128)
    o = z(1, 8192, 32, 128)
    a = make_args(q, q, q, q, z(1, 8192, 32), None, None, None, o, None)
    assert kda_fwd_workspace_bytes(a) > KDA_NO_ALLOC_MAX_BYTES
    o.fill_(1.0)
    assert load_library().kda_fwd_no_alloc(ctypes.byref(a)) == KDA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((o == 1.0).all())    # nothing was launched
