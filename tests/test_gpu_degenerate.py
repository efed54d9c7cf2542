"""Degenerate inputs of the method on the GPU path, through the C ABI, against the
token recurrence (bar max|x - x_ref| / max|x_ref| <= 1e-2, outputs pre-filled with
NaN): no write (beta = 0: the state only decays), full-strength writes (beta = 1),
no decay (g = 0: the ungated delta rule, every gate factor exactly 1), both at once,
zero keys (nothing is written or erased), zero values, and single-token sequences.
Each runs on the library's scan choice, on forced segments and at chunk 16."""
import numpy as np
import pytest

from synth.inputs import make_inputs
from oracle import recurrent

from _gpu_util import FIELDS, nerr, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-2
OPTS = [{}, {"seg_chunks": 1}, {"chunk": 16}]
IDS = ["plan", "seg1", "chunk16"]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


def run_and_check(d, opts, expect_zero_o=False):
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    t = to_device(d)
    N = t["q"].shape[0] if t["cu_seqlens"] is None else t["cu_seqlens"].numel() - 1
    o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device=t["v"].device)
    ht = torch.full((N, t["v"].shape[2], t["q"].shape[3], t["v"].shape[3]), float("nan"),
                    dtype=torch.float32, device=t["v"].device)
    kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"],
            cu_seqlens=t["cu_seqlens"], o=o, ht=ht, **opts)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    ht = ht.cpu().numpy().astype(np.float64)
    o_ref, ht_ref = recurrent(**{k: d[k] for k in FIELDS}, scale=d["scale"], h0=d["h0"],
                              cu_seqlens=d["cu_seqlens"])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    if expect_zero_o:
        assert np.all(o == 0) and np.all(o_ref == 0) and np.all(ht == 0) and np.all(ht_ref == 0)
    else:
        eo = nerr(o, o_ref)
        print(f"  o {eo:.2e}", flush=True)
        assert eo <= TOL
    eh = nerr(ht, ht_ref)
    print(f"  ht {eh:.2e}", flush=True)
    assert eh <= TOL
    return o, ht


def base(seed, T=64 * 3 + 11, has_h0=True):
    return make_inputs(seed, B=2, T=T, HQK=1, HV=2, K=128, V=64, has_h0=has_h0)


@pytest.mark.parametrize("opts", OPTS, ids=IDS)
def test_no_write_state_only_decays(opts):
    d = base(800)
    d["beta"] = np.zeros_like(d["beta"])
    o, ht = run_and_check(d, opts)
    # beta = 0 leaves h0 decayed by the whole gate sum: ht = exp(sum_t g_t) h0 per key row
    decay = np.exp(d["g"].sum(axis=1))                      # [B, HV, K]
    assert nerr(ht, decay[..., None] * d["h0"]) <= TOL


@pytest.mark.parametrize("opts", OPTS, ids=IDS)
def test_full_strength_writes(opts):
    d = base(801)
    d["beta"] = np.ones_like(d["beta"])
    run_and_check(d, opts)


@pytest.mark.parametrize("opts", OPTS, ids=IDS)
def test_no_decay_ungated_delta_rule(opts):
    d = base(802)
    d["g"] = np.zeros_like(d["g"])
    run_and_check(d, opts)


@pytest.mark.parametrize("opts", OPTS, ids=IDS)
def test_no_decay_and_full_strength(opts):
    d = base(803)
    d["g"] = np.zeros_like(d["g"])
    d["beta"] = np.ones_like(d["beta"])
    run_and_check(d, opts)


@pytest.mark.parametrize("opts", OPTS, ids=IDS)
def test_zero_keys_write_nothing(opts):
    # k = 0: no write and no erase, so with h0 = 0 the state and the outputs stay zero
    d = base(804, has_h0=False)
    d["k"] = np.zeros_like(d["k"])
    run_and_check(d, opts, expect_zero_o=True)


@pytest.mark.parametrize("opts", OPTS, ids=IDS)
def test_zero_values_from_zero_state(opts):
    d = base(805, has_h0=False)
    d["v"] = np.zeros_like(d["v"])
    run_and_check(d, opts, expect_zero_o=True)


@pytest.mark.parametrize("opts", OPTS, ids=IDS)
def test_single_token_sequences(opts):
    d = make_inputs(806, B=1, T=0, HQK=1, HV=2, K=128, V=64, has_h0=True, lengths=[1, 1, 1, 0, 1])
    run_and_check(d, opts)


@pytest.mark.parametrize("opts", OPTS, ids=IDS)
@pytest.mark.parametrize("has_h0", [True, False])
def test_fixed_length_without_tokens(opts, has_h0):
    # B sequences of T = 0 tokens: no o rows, and each final state is its initial state
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    d = make_inputs(807, B=2, T=0, HQK=1, HV=2, K=128, V=64, has_h0=has_h0)
    t = to_device(d)
    ht = torch.full((2, 2, 128, 64), float("nan"), dtype=torch.float32, device="cuda")
    o, ht = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"], ht=ht, **opts)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64)
    want = d["h0"] if has_h0 else np.zeros((2, 2, 128, 64), np.float32)
    assert np.array_equal(ht.cpu().numpy(), want)


@pytest.mark.parametrize("seg", [0, 2])
def test_backward_without_tokens(seg):
    # T = 0: no dv2 rows, no checkpoints, and dh0 is dht
    import torch
    from gated_delta_rule_chunked_amd import kda_bwd_dhu
    bf = torch.bfloat16
    e = lambda *s, dt=bf: torch.empty(s, dtype=dt, device="cuda")
    dht = torch.randn((2, 2, 128, 64), device="cuda")
    dv2, dhc, dh0 = kda_bwd_dhu(e(2, 0, 2, 128), e(2, 0, 2, 128), e(2, 0, 2, 128), e(2, 0, 2, 128, dt=torch.float32),
                                e(2, 0, 2, 64), e(2, 0, 2, 64), dht, scale=0.1, seg_chunks=seg)
    torch.cuda.synchronize()
    assert dv2.shape == (2, 0, 2, 64) and dhc.shape[0] == 0
    assert torch.equal(dh0, dht)
