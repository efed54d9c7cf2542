"""Pins for the oracle's backward state scan (``bwd_dhu`` via ``backward_states``).

The loss L = <do, o> + <dht, ht> of the token recurrence O1 (``recurrent``, code
independent of the chunked form) is affine in h0, in v and in the state at any
token boundary, so finite differences along a direction D are exact up to fp64
rounding:
    <dh0, D>          = L(h0 + D) - L(h0)
    <dL/dv, D>        = L(v + D) - L(v),      dL/dv = (Tm diag beta)^T dv2 per chunk
    <dhc[c], D>       = L_suffix(S_c + D) - L_suffix(S_c)   (O1 re-run after chunk c)
Planted mistakes in a copy of the stage are caught by these pins.
"""
import numpy as np
import pytest

import oracle.kda_oracle as ko
from oracle import backward_states, chunked, recurrent
from synth.inputs import make_inputs

FIELDS = ("q", "k", "v", "g", "beta")


def case(seed=31, chunk=16):
    d = make_inputs(seed, B=1, T=0, HQK=1, HV=2, K=8, V=6, has_h0=True, lengths=[40, 0, 17, 70])
    rng = np.random.default_rng(seed + 1000)
    do = rng.standard_normal(d["v"].shape)
    dht = rng.standard_normal(d["h0"].shape)
    return d, do, dht, chunk


def loss(d, do, dht, **over):
    a = {k: over.get(k, d[k]) for k in FIELDS}
    o, ht = recurrent(**a, scale=d["scale"], h0=over.get("h0", d["h0"]), cu_seqlens=d["cu_seqlens"])
    return float(np.sum(do * o) + np.sum(dht * ht))


def rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


def check_pins(d, do, dht, chunk):
    dv2, dhc, dh0 = backward_states(*(d[k] for k in FIELDS), d["scale"], do, dht=dht,
                                    cu_seqlens=d["cu_seqlens"], chunk=chunk)
    rng = np.random.default_rng(5)
    L0 = loss(d, do, dht)
    # dh0
    for _ in range(2):
        D = rng.standard_normal(d["h0"].shape)
        assert rel(np.sum(dh0 * D), loss(d, do, dht, h0=d["h0"] + D) - L0) < 1e-8
    # dv2 through dL/dv = TmB^T dv2
    _, _, inter = chunked(*(d[k] for k in FIELDS), d["scale"], h0=d["h0"], cu_seqlens=d["cu_seqlens"],
                          chunk=chunk, return_intermediates=True)
    dLdv = np.zeros_like(d["v"], dtype=np.float64)
    beta = np.asarray(d["beta"], dtype=np.float64)
    for ci in inter:
        r0, L = ci["row0"], ci["rows"]
        TmB = ci["Tm"] * beta[0, r0:r0 + L].T[:, None, :]
        dLdv[0, r0:r0 + L] = np.einsum("hij,ihv->jhv", TmB, dv2[0, r0:r0 + L])
    for _ in range(2):
        D = rng.standard_normal(d["v"].shape)
        assert rel(np.sum(dLdv * D), loss(d, do, dht, v=np.asarray(d["v"], np.float64) + D) - L0) < 1e-8
    # dhc: gradient of the state after each chunk, by re-running O1 on the suffix
    _, _, states = recurrent(*(d[k] for k in FIELDS), d["scale"], h0=d["h0"], cu_seqlens=d["cu_seqlens"],
                             return_states=True)
    cu = [int(x) for x in d["cu_seqlens"]]
    assert len(dhc) == len(inter)
    for c, ci in enumerate(inter):
        n, r1 = ci["seq"], ci["row0"] + ci["rows"]
        S = states[0, r1 - 1]
        sub = {k: np.asarray(d[k], np.float64)[:, r1:cu[n + 1]] for k in FIELDS}
        D = rng.standard_normal(S.shape)
        def Ls(h):
            o, ht = recurrent(**sub, scale=d["scale"], h0=h[None])
            return float(np.sum(do[:, r1:cu[n + 1]] * o) + np.sum(dht[n] * ht[0]))
        assert rel(np.sum(dhc[c] * D), Ls(S + D) - Ls(S)) < 1e-8, c
    return dv2, dhc, dh0


def test_backward_states_match_finite_differences_of_recurrence():
    check_pins(*case())


def test_dh0_does_not_depend_on_chunk_size():
    d, do, dht, _ = case(seed=33)
    ref = backward_states(*(d[k] for k in FIELDS), d["scale"], do, dht=dht, cu_seqlens=d["cu_seqlens"], chunk=1)[2]
    for C in (7, 16, 64):
        dh0 = backward_states(*(d[k] for k in FIELDS), d["scale"], do, dht=dht, cu_seqlens=d["cu_seqlens"],
                              chunk=C)[2]
        assert np.abs(dh0 - ref).max() < 1e-10 * np.abs(ref).max()


MUTANTS = {
    "no_scale": lambda qg, kg, w, gcum, do, dv_in, scale, **kw: GOOD(qg, kg, w, gcum, do, dv_in, 1.0, **kw),
    "no_decay": lambda qg, kg, w, gcum, do, dv_in, scale, **kw: GOOD(qg, kg, w, 0 * gcum, do, dv_in, scale, **kw),
    "w_sign": lambda qg, kg, w, gcum, do, dv_in, scale, **kw: GOOD(qg, kg, -np.asarray(w), gcum, do, dv_in, scale, **kw),
    "no_dv_in": lambda qg, kg, w, gcum, do, dv_in, scale, **kw: GOOD(qg, kg, w, gcum, do, 0 * dv_in, scale, **kw),
    "first_row_decay": lambda qg, kg, w, gcum, do, dv_in, scale, **kw: GOOD(
        qg, kg, w, np.roll(gcum, 1, axis=1), do, dv_in, scale, **kw),
}
GOOD = ko.bwd_dhu


@pytest.mark.parametrize("kind", sorted(MUTANTS))
def test_bwd_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(ko, "bwd_dhu", MUTANTS[kind])
    with pytest.raises(AssertionError):
        check_pins(*case())
