"""The output scale as an argument, through the C ABI: every other parity case runs at
scale = K^-0.5, which a kernel could reproduce without reading the argument.  Here the
forward (its scan choice at this shape, forced segments, chunk 16) and the backward
state scan (serial and segmented) run at other scales, against the oracle at the same
scale; bar max|x - x_ref| / max|x_ref| <= 1e-2."""
import numpy as np
import pytest

from synth.inputs import make_grads, make_inputs
from oracle import recurrent

from _gpu_util import FIELDS, nerr, run_hip
from test_gpu_bwd import check, reference, run_gpu, scan_inputs

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


@pytest.mark.parametrize("opts", [{}, {"seg_chunks": 2}, {"chunk": 16}], ids=["plan", "seg2", "chunk16"])
@pytest.mark.parametrize("scale", [0.37, 1.0, 0.02])
def test_forward_scale_argument(scale, opts):
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    from _gpu_util import to_device
    d = dict(make_inputs(700, B=2, T=64 * 3 + 29, HQK=1, HV=2, K=128, V=64, has_h0=True), scale=scale)
    t = to_device(d)
    o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device=t["v"].device)
    o, ht = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=scale, h0=t["h0"], o=o, **opts)
    torch.cuda.synchronize()
    o_ref, ht_ref = recurrent(**{k: d[k] for k in FIELDS}, scale=scale, h0=d["h0"])
    eo = nerr(o.float().cpu().numpy().astype(np.float64), o_ref)
    eh = nerr(ht.cpu().numpy().astype(np.float64), ht_ref)
    print(f"  scale {scale} {opts}: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert eo <= TOL and eh <= TOL


def test_forward_output_is_linear_in_scale():
    # o is linear in the scale (ht does not depend on it): 1.0 and 0.25 give o in a
    # ratio of 4 up to bf16 rounding, and the same ht bit for bit
    d = make_inputs(701, B=1, T=150, HQK=1, HV=2, K=64, V=32, has_h0=True)
    o1, h1 = run_hip(dict(d, scale=1.0))
    o2, h2 = run_hip(dict(d, scale=0.25))
    assert np.array_equal(h1, h2)
    assert nerr(4.0 * o2, o1) <= 1e-2


@pytest.mark.parametrize("seg", [0, 2])
@pytest.mark.parametrize("scale", [0.37, 1.0])
def test_backward_scale_argument(scale, seg):
    d = dict(make_inputs(702, B=1, T=64 * 4 + 21, HQK=1, HV=2, K=128, V=64, has_h0=False), scale=scale)
    gr = make_grads(d, 7020)
    x = scan_inputs(d, gr)
    check(run_gpu(x, d, seg_chunks=seg), reference(x, d), f"scale {scale} seg {seg}")
