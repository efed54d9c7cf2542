"""The seeded input generator: deterministic, bf16-exact, the stated distributions."""
import numpy as np

from synth import CONFIGS, make_config_inputs, round_to_bf16, bf16_bits
from synth.inputs import make_inputs


def test_round_to_bf16_is_rne():
    # 1 + 2^-8 is exactly halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert round_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 1 + 2^-6
    assert round_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert round_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7
    x = np.random.default_rng(0).standard_normal(10000)
    r = round_to_bf16(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8)
    bf16_bits(r)  # exactly representable


def test_deterministic_and_bf16_exact():
    a = make_config_inputs(1)
    b = make_config_inputs(1)
    for k in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(a[k], b[k])
        bf16_bits(a[k])
    assert a["h0"] is None and a["cu_seqlens"] is None


def test_distributions():
    d = make_inputs(2, B=2, T=512, HQK=2, HV=4, K=128, V=64, has_h0=True)
    assert d["q"].shape == (2, 512, 2, 128) and d["v"].shape == (2, 512, 4, 64)
    assert d["g"].shape == (2, 512, 4, 128) and d["beta"].shape == (2, 512, 4)
    assert d["h0"].shape == (2, 4, 128, 64) and d["h0"].dtype == np.float32
    nq = np.linalg.norm(d["q"].astype(np.float64), axis=-1)
    assert np.all(np.abs(nq - 1) < 1e-2)
    assert np.all(d["g"] < 0) and abs(d["g"].mean() + 0.18) < 0.02
    assert np.all((d["beta"] > 0) & (d["beta"] < 1)) and abs(d["beta"].mean() - 0.5) < 0.02
    assert abs(d["h0"].std() - 0.1) < 0.01
    assert abs(d["scale"] - 128 ** -0.5) < 1e-15


def test_varlen_lengths_seeded():
    w = CONFIGS[4]
    rng = np.random.default_rng(w.seed)
    lengths = rng.integers(*w.varlen_range, size=w.n_varlen)
    d = make_inputs(w.seed, 1, 0, 1, 1, 8, 8, True, n_varlen=w.n_varlen, varlen_range=w.varlen_range)
    assert np.array_equal(np.diff(d["cu_seqlens"]), lengths)
    assert np.all((lengths >= 64) & (lengths <= 4096))
    assert d["h0"].shape[0] == 16
