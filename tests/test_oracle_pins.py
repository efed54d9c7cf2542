"""Pins for the fp64 CPU oracle: closed forms, invariants, brute force and the
chunk-table example printed on the FlashKDA walkthrough page.

Each ``pin_*`` takes the recurrence under test (signature of
``oracle.recurrent``) so that ``test_pins_catch_planted_mistakes`` can run the
same pins against deliberately broken copies of the recurrence and check that
every planted mistake is caught.  No GPU involved.
"""
import json
import os

import numpy as np
import pytest

from oracle import chunk_lengths, chunk_table, chunked, recurrent
from synth.inputs import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def nerr(a, b):
    """max |a - b| / max |b| (the normalised max error used throughout)."""
    a, b = np.asarray(a), np.asarray(b)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def small(seed=11, T=40, K=8, V=6, HV=2, HQK=1, h0=True, **kw):
    d = make_inputs(seed, B=1, T=T, HQK=HQK, HV=HV, K=K, V=V, has_h0=h0, **kw)
    args = {k: d[k].astype(np.float64) for k in ("q", "k", "v", "g", "beta")}
    return d, args


def fp64_inputs(seed, T, K, V, HV=1, B=1, unit_k=True, g_scale=1.0):
    """Unrounded float64 inputs (for identities that need exact unit-norm keys)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, HV, K))
    k = rng.standard_normal((B, T, HV, K))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, HV, V))
    beta = rng.uniform(0.05, 1.0, size=(B, T, HV))
    g = -g_scale * rng.uniform(0.0, 0.5, size=(B, T, HV, K))
    h0 = rng.standard_normal((B, HV, K, V))
    return dict(q=q, k=k, v=v, g=g, beta=beta), h0


# --------------------------------------------------------------------- pins


def pin_rank1_matches_matrix_form(rec):
    """S_t == (I - b k k^T) diag(e^g) S_{t-1} + b k v^T, with explicit K x K matrices."""
    d, a = small(seed=3, T=24, K=6, V=5, HV=1, HQK=1)
    h0 = d["h0"].astype(np.float64)
    _, _, S = rec(**a, scale=d["scale"], h0=h0, return_states=True)
    prev = h0[0, 0]
    for t in range(a["q"].shape[1]):
        kt, vt, bt = a["k"][0, t, 0], a["v"][0, t, 0], a["beta"][0, t, 0]
        M = np.eye(len(kt)) - bt * np.outer(kt, kt)
        want = M @ np.diag(np.exp(a["g"][0, t, 0])) @ prev + bt * np.outer(kt, vt)
        assert nerr(S[0, t, 0], want) < 1e-13
        prev = want


def pin_single_token_closed_form(rec):
    """T = 1: o = scale * S_1^T q with S_1 = (I - b k k^T) diag(e^g) h0 + b k v^T;
    with h0 = 0 this is o = scale * b (q . k) v."""
    d, a = small(seed=5, T=1, K=8, V=6, HV=1, HQK=1)
    h0 = d["h0"].astype(np.float64)
    o, ht = rec(**a, scale=d["scale"], h0=h0)
    q, k, v, b, g = (a[x][0, 0, 0] for x in ("q", "k", "v", "beta", "g"))
    S1 = (np.eye(8) - b * np.outer(k, k)) @ (np.exp(g)[:, None] * h0[0, 0]) + b * np.outer(k, v)
    assert nerr(ht[0, 0], S1) < 1e-14
    assert nerr(o[0, 0, 0], d["scale"] * S1.T @ q) < 1e-14
    o0, _ = rec(**a, scale=d["scale"], h0=None)
    assert nerr(o0[0, 0, 0], d["scale"] * b * (q @ k) * v) < 1e-14


def pin_beta_zero_pure_decay(rec):
    """beta = 0: nothing is erased or written, S_t = diag(exp G_t) h0 with G the
    inclusive cumsum of g, and o_t = scale * S_t^T q_t."""
    d, a = small(seed=6, T=30, K=8, V=5, HV=2, HQK=2)
    a["beta"] = np.zeros_like(a["beta"])
    h0 = d["h0"].astype(np.float64)
    o, ht = rec(**a, scale=d["scale"], h0=h0)
    G = np.cumsum(a["g"][0], axis=0)                       # [T, HV, K]
    for t in range(30):
        for h in range(2):
            St = np.exp(G[t, h])[:, None] * h0[0, h]
            assert nerr(o[0, t, h], d["scale"] * St.T @ a["q"][0, t, h]) < 1e-13
    assert nerr(ht[0], np.exp(G[-1])[:, :, None] * h0[0]) < 1e-13


def pin_write_exactness_ungated(rec):
    """g = 0, beta = 1, unit-norm k (ungated delta rule): after each token the
    memory returns exactly the value just written, k_t^T S_t = v_t."""
    a, h0 = fp64_inputs(7, T=20, K=8, V=5)
    a["g"] = np.zeros_like(a["g"])
    a["beta"] = np.ones_like(a["beta"])
    _, _, S = rec(**a, scale=0.3, h0=h0, return_states=True)
    for t in range(20):
        assert nerr(a["k"][0, t, 0] @ S[0, t, 0], a["v"][0, t, 0]) < 1e-13


def pin_write_identity_general(rec):
    """Any gate: k_t^T S_t = (1 - b|k|^2) k_t^T diag(e^g_t) S_{t-1} + b|k|^2 v_t.
    Holds for decay-then-erase; erase-then-decay breaks it when K > 1."""
    a, h0 = fp64_inputs(8, T=20, K=8, V=5, unit_k=False)
    _, _, S = rec(**a, scale=0.3, h0=h0, return_states=True)
    prev = h0[0, 0]
    for t in range(20):
        k, v, b, g = (a[x][0, t, 0] for x in ("k", "v", "beta", "g"))
        kk = k @ k
        want = (1 - b * kk) * (k @ (np.exp(g)[:, None] * prev)) + b * kk * v
        assert nerr(k @ S[0, t, 0], want) < 1e-12
        prev = S[0, t, 0]


def pin_one_hot_gla_closed_form(rec):
    """Distinct one-hot keys, h0 = 0: the erase term vanishes and the method is
    gated linear attention, o_t = scale * sum_{s<=t} b_s q_t[i_s] e^{G_t[i_s]-G_s[i_s]} v_s."""
    T, K, V = 10, 12, 4
    rng = np.random.default_rng(9)
    idx = rng.permutation(K)[:T]
    a, _ = fp64_inputs(9, T=T, K=K, V=V)
    a["k"] = np.zeros_like(a["k"])
    a["k"][0, np.arange(T), 0, idx] = 1.0
    o, _ = rec(**a, scale=0.7, h0=None)
    G = np.cumsum(a["g"][0, :, 0], axis=0)                  # [T, K]
    for t in range(T):
        want = np.zeros(V)
        for s in range(t + 1):
            i = idx[s]
            want += a["beta"][0, s, 0] * a["q"][0, t, 0, i] * np.exp(G[t, i] - G[s, i]) * a["v"][0, s, 0]
        assert nerr(o[0, t, 0], 0.7 * want) < 1e-13


def pin_repeated_one_hot_overwrite(rec):
    """beta = 1, g = 0, the same one-hot key every token: row i of the state is
    overwritten by the latest value and every other row keeps h0."""
    T, K, V, i = 6, 5, 3, 2
    a, h0 = fp64_inputs(10, T=T, K=K, V=V)
    a["g"] = np.zeros_like(a["g"])
    a["beta"] = np.ones_like(a["beta"])
    a["k"] = np.zeros_like(a["k"])
    a["k"][0, :, 0, i] = 1.0
    _, _, S = rec(**a, scale=1.0, h0=h0, return_states=True)
    for t in range(T):
        assert nerr(S[0, t, 0, i], a["v"][0, t, 0]) < 1e-14
        rest = [r for r in range(K) if r != i]
        assert np.array_equal(S[0, t, 0, rest], h0[0, 0, rest])


def pin_strong_decay_limit(rec):
    """g = -60: the old state is forgotten every token, so
    o_t = scale * b_t (q_t . k_t) v_t up to e^-60."""
    d, a = small(seed=12, T=16, K=8, V=5, HV=1, HQK=1)
    a["g"] = np.full_like(a["g"], -60.0)
    o, _ = rec(**a, scale=d["scale"], h0=d["h0"].astype(np.float64))
    want = d["scale"] * (a["beta"][..., None] * np.sum(a["q"] * a["k"], -1, keepdims=True) * a["v"])
    assert np.abs(o - want).max() < 1e-20


def pin_linearity(rec):
    """(v, h0) -> (o, ht) is linear; o is linear in scale; ht depends on neither q nor scale."""
    d, a = small(seed=13, T=20, K=6, V=5, HV=2, HQK=1)
    h0 = d["h0"].astype(np.float64)
    rng = np.random.default_rng(0)
    v2, h2 = rng.standard_normal(a["v"].shape), rng.standard_normal(h0.shape)
    o1, t1 = rec(**a, scale=0.5, h0=h0)
    o2, t2 = rec(**{**a, "v": v2}, scale=0.5, h0=h2)
    o3, t3 = rec(**{**a, "v": 2 * a["v"] - 3 * v2}, scale=0.5, h0=2 * h0 - 3 * h2)
    assert nerr(o3, 2 * o1 - 3 * o2) < 1e-12 and nerr(t3, 2 * t1 - 3 * t2) < 1e-12
    o4, t4 = rec(**{**a, "q": rng.standard_normal(a["q"].shape)}, scale=1.5, h0=h0)
    assert np.array_equal(t4, t1)
    o5, _ = rec(**a, scale=1.5, h0=h0)
    assert nerr(o5, 3 * o1) < 1e-14


def pin_causality(rec):
    """Changing rows after t leaves o[:t+1] bit-identical."""
    d, a = small(seed=14, T=30, K=6, V=5, HV=2, HQK=2)
    o1, _ = rec(**a, scale=d["scale"])
    b = {k: x.copy() for k, x in a.items()}
    rng = np.random.default_rng(1)
    for x in ("q", "k", "v", "g"):
        b[x][0, 17:] = rng.standard_normal(b[x][0, 17:].shape) - (2.0 if x == "g" else 0.0)
    b["beta"][0, 17:] = 0.9
    o2, _ = rec(**b, scale=d["scale"])
    assert np.array_equal(o1[0, :17], o2[0, :17])
    assert not np.allclose(o1[0, 17:], o2[0, 17:])


def pin_split_resume(rec):
    """Run [0, T1) then [T1, T) from its final state == one run over [0, T)."""
    d, a = small(seed=15, T=50, K=6, V=5, HV=2, HQK=1)
    h0 = d["h0"].astype(np.float64)
    o, ht = rec(**a, scale=d["scale"], h0=h0)
    first = {k: x[:, :21] for k, x in a.items()}
    second = {k: x[:, 21:] for k, x in a.items()}
    oa, ha = rec(**first, scale=d["scale"], h0=h0)
    ob, hb = rec(**second, scale=d["scale"], h0=ha)
    assert nerr(np.concatenate([oa, ob], axis=1), o) < 1e-12 and nerr(hb, ht) < 1e-12


def pin_varlen_equals_separate(rec):
    """A packed varlen batch (including an empty sequence) equals separate runs,
    each from its own h0; an empty sequence returns its h0 unchanged."""
    lengths = [9, 0, 17, 5]
    d, a = small(seed=16, K=6, V=5, HV=2, HQK=1, lengths=lengths)
    cu, h0 = d["cu_seqlens"], d["h0"].astype(np.float64)
    o, ht = rec(**a, scale=d["scale"], h0=h0, cu_seqlens=cu)
    for n in range(len(lengths)):
        s = slice(cu[n], cu[n + 1])
        part = {k: x[:, s] for k, x in a.items()}
        on, hn = rec(**part, scale=d["scale"], h0=h0[n:n + 1])
        if lengths[n]:
            assert nerr(o[:, s], on) < 1e-14
        assert nerr(ht[n], hn[0]) < 1e-14
    assert np.array_equal(ht[1], h0[1])


def pin_gva_equals_repeated_heads(rec):
    """Grouped heads (HV = 2 HQK): value heads 2i, 2i+1 read q/k head i, so the run
    equals the ungrouped run with q, k repeated per value head."""
    d, a = small(seed=17, T=20, K=6, V=5, HV=4, HQK=2)
    o, ht = rec(**a, scale=d["scale"], h0=d["h0"])
    rep = dict(a, q=np.repeat(a["q"], 2, axis=2), k=np.repeat(a["k"], 2, axis=2))
    o2, ht2 = rec(**rep, scale=d["scale"], h0=d["h0"])
    assert np.array_equal(o, o2) and np.array_equal(ht, ht2)
    # and not some other grouping
    alt = dict(a, q=np.tile(a["q"], (1, 1, 2, 1)), k=np.tile(a["k"], (1, 1, 2, 1)))
    o3, _ = rec(**alt, scale=d["scale"], h0=d["h0"])
    assert not np.allclose(o, o3)


def pin_norm_bound(rec):
    """With beta in [0,1] and |k| <= 1 the transition has spectral norm <= 1, so
    |S_T|_2 <= |h0|_2 + sum_t beta_t |k_t| |v_t|."""
    d, a = small(seed=18, T=60, K=8, V=6, HV=1, HQK=1)
    h0 = d["h0"].astype(np.float64)
    _, ht = rec(**a, scale=d["scale"], h0=h0)
    bound = np.linalg.norm(h0[0, 0], 2) + np.sum(
        a["beta"][0, :, 0] * np.linalg.norm(a["k"][0, :, 0], axis=-1) * np.linalg.norm(a["v"][0, :, 0], axis=-1))
    assert np.linalg.norm(ht[0, 0], 2) <= bound * (1 + 1e-12)


PINS = [pin_rank1_matches_matrix_form, pin_single_token_closed_form, pin_beta_zero_pure_decay,
        pin_write_exactness_ungated, pin_write_identity_general, pin_one_hot_gla_closed_form,
        pin_repeated_one_hot_overwrite, pin_strong_decay_limit, pin_linearity, pin_causality,
        pin_split_resume, pin_varlen_equals_separate, pin_gva_equals_repeated_heads, pin_norm_bound]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_recurrent_pin(pin):
    pin(recurrent)


# ------------------------------------------------- chunked form vs recurrence


@pytest.mark.parametrize("C", [1, 7, 16, 64, 100, 200])
def test_chunked_matches_recurrent(C):
    d, a = small(seed=21, T=200, K=16, V=12, HV=2, HQK=1)
    o1, h1 = recurrent(**a, scale=d["scale"], h0=d["h0"])
    o2, h2 = chunked(**a, scale=d["scale"], h0=d["h0"], chunk=C)
    assert nerr(o2, o1) < 1e-10 and nerr(h2, h1) < 1e-10


@pytest.mark.parametrize("C", [16, 64])
def test_chunked_matches_recurrent_config1(C):
    from synth import make_config_inputs
    d = make_config_inputs(1)
    a = {k: d[k] for k in ("q", "k", "v", "g", "beta")}
    o1, h1 = recurrent(**a, scale=d["scale"])
    o2, h2 = chunked(**a, scale=d["scale"], chunk=C)
    assert nerr(o2, o1) < 1e-10 and nerr(h2, h1) < 1e-10


@pytest.mark.parametrize("C", [16, 64])
def test_chunked_matches_recurrent_varlen_gva(C):
    d, a = small(seed=22, K=16, V=8, HV=4, HQK=2, lengths=[70, 0, 129, 1, 64])
    o1, h1 = recurrent(**a, scale=d["scale"], h0=d["h0"], cu_seqlens=d["cu_seqlens"])
    o2, h2 = chunked(**a, scale=d["scale"], h0=d["h0"], cu_seqlens=d["cu_seqlens"], chunk=C)
    assert nerr(o2, o1) < 1e-10 and nerr(h2, h1) < 1e-10


@pytest.mark.parametrize("C", [16, 64])
def test_chunk_start_states_match_recurrent_states(C):
    """The per-chunk states of the chunked form (the state before each chunk) are
    the token recurrence's state after the chunk's previous token, or h0 at each
    sequence start (varlen with empty and one-token sequences, GVA)."""
    d, a = small(seed=23, K=16, V=8, HV=4, HQK=2, lengths=[70, 0, 129, 1, 64])
    _, _, states = recurrent(**a, scale=d["scale"], h0=d["h0"], cu_seqlens=d["cu_seqlens"], return_states=True)
    _, _, inter = chunked(**a, scale=d["scale"], h0=d["h0"], cu_seqlens=d["cu_seqlens"], chunk=C,
                          return_intermediates=True)
    cu = [int(x) for x in d["cu_seqlens"]]
    n_chunks = sum(-(-(cu[i + 1] - cu[i]) // C) for i in range(len(cu) - 1))
    assert len(inter) == n_chunks
    for ci in inter:
        n, r0 = ci["seq"], ci["row0"]
        ref = d["h0"][n] if r0 == cu[n] else states[0, r0 - 1]
        assert nerr(ci["h"], ref) < 1e-12, (n, r0)


def test_chunk_intermediates_definitions():
    """The intra-stage pieces satisfy their defining relations: Tm (I + Akk) = I,
    Aqk is lower triangular with scale * q_i . k_i on the diagonal, and the
    chunk's final state is diag(e^G) h0 + kg^T (u - w h0) (brute-force recurrence)."""
    d, a = small(seed=23, T=64, K=8, V=6, HV=1, HQK=1)
    h0 = d["h0"].astype(np.float64)
    _, _, inter = chunked(**a, scale=d["scale"], h0=h0, chunk=64, return_intermediates=True)
    ci = inter[0]
    eye = np.eye(64)
    assert nerr(ci["Tm"][0] @ (eye + ci["Akk"][0]), eye) < 1e-12
    assert np.all(np.triu(ci["Aqk"][0], 1) == 0) and np.all(np.triu(ci["Akk"][0]) == 0)
    diag = d["scale"] * np.sum(a["q"][0, :, 0] * a["k"][0, :, 0], -1)
    assert nerr(np.diag(ci["Aqk"][0]), diag) < 1e-14
    _, ht = recurrent(**a, scale=d["scale"], h0=h0)
    vp = ci["u"][:, 0] - ci["w"][:, 0] @ h0[0, 0]
    assert nerr(np.exp(ci["gd"][0])[:, None] * h0[0, 0] + ci["kg"][:, 0].T @ vp, ht[0, 0]) < 1e-12


# -------------------------------------------------------------- chunk table


def test_chunk_table_matches_flashkda_examples():
    ex = json.load(open(os.path.join(GOLDEN, "flashkda_chunk_table.json")))["examples"]
    t = ex[0]
    base, tiles = chunk_table(t["lengths"], t["chunk"])
    assert base == t["tile_base"] and tiles == t["t_tiles"]
    cu = np.concatenate([[0], np.cumsum(t["lengths"])])
    assert list(cu[:-1]) == t["bos"] and list(cu[1:]) == t["eos"]
    tail = ex[1]
    rows = chunk_lengths(tail["lengths"][0], tail["chunk"])
    assert rows == tail["chunk_rows"]
    assert list(np.cumsum([0] + rows[:-1])) == tail["first_row"]


# ------------------------------------------- the pins have teeth (mutants)


def _mutant(kind):
    """A copy of the recurrence with one planted mistake."""
    def rec(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, return_states=False):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        B, T, HQK, K = q.shape
        HV, V = v.shape[2], v.shape[3]
        hq = (np.arange(HV) % HQK) if kind == "head_map" else np.arange(HV) // (HV // HQK)
        cu = [0, T] if cu_seqlens is None else list(cu_seqlens)
        seqs = [(b, 0, T) for b in range(B)] if cu_seqlens is None else \
            [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
        o = np.zeros((B, T, HV, V))
        ht = np.zeros((len(seqs), HV, K, V))
        states = np.zeros((B, T, HV, K, V))
        for n, (b, bos, eos) in enumerate(seqs):
            S = np.zeros((HV, K, V)) if h0 is None else np.array(h0[n], dtype=np.float64)
            for t in range(bos, eos):
                kt, qt, vt, bt = k[b, t][hq], q[b, t][hq], v[b, t], beta[b, t]
                D = np.exp(g[b, t])[:, :, None]
                if kind == "erase_before_decay":
                    S = S + bt[:, None, None] * kt[:, :, None] * (vt - np.einsum("hkv,hk->hv", S, kt))[:, None, :]
                    S = D * S
                    o[b, t] = scale * np.einsum("hkv,hk->hv", S, qt)
                elif kind == "read_before_write":
                    S = D * S
                    o[b, t] = scale * np.einsum("hkv,hk->hv", S, qt)
                    S = S + bt[:, None, None] * kt[:, :, None] * (vt - np.einsum("hkv,hk->hv", S, kt))[:, None, :]
                elif kind == "no_beta_on_write":
                    S = D * S
                    S = S - bt[:, None, None] * kt[:, :, None] * np.einsum("hkv,hk->hv", S, kt)[:, None, :] \
                        + kt[:, :, None] * vt[:, None, :]
                    o[b, t] = scale * np.einsum("hkv,hk->hv", S, qt)
                elif kind == "gate_sign":
                    S = np.exp(-g[b, t])[:, :, None] * S
                    S = S + bt[:, None, None] * kt[:, :, None] * (vt - np.einsum("hkv,hk->hv", S, kt))[:, None, :]
                    o[b, t] = scale * np.einsum("hkv,hk->hv", S, qt)
                else:  # "transposed_readout" and "head_map"
                    S = D * S
                    S = S + bt[:, None, None] * kt[:, :, None] * (vt - np.einsum("hkv,hk->hv", S, kt))[:, None, :]
                    if kind == "transposed_readout" and K == V:
                        o[b, t] = scale * np.einsum("hkv,hv->hk", S, qt)
                    else:
                        o[b, t] = scale * np.einsum("hkv,hk->hv", S, qt)
                states[b, t] = S
            ht[n] = S
        return (o, ht, states) if return_states else (o, ht)
    return rec


def _caught(rec):
    for pin in PINS:
        try:
            pin(rec)
        except (AssertionError, ValueError, IndexError):
            return pin.__name__
    return None


@pytest.mark.parametrize("kind", ["erase_before_decay", "read_before_write", "no_beta_on_write",
                                  "gate_sign", "head_map"])
def test_pins_catch_planted_mistakes(kind):
    assert _caught(_mutant(kind)) is not None, f"no pin caught mutant {kind}"


def test_clean_copy_passes_pins():
    assert _caught(_mutant("none")) is None


def test_gate_floor_changes_the_recurrence_by_less_than_its_decay():
    """The GPU path raises per-token gates below -10 to -10.  In exact arithmetic
    that changes the outputs by at most about exp(-10) = 4.5e-5 of the state
    magnitude: checked here on the token recurrence with whole tokens, whole 16-token
    blocks, single dimensions and -inf gates below the floor."""
    d = make_inputs(43, B=1, T=200, HQK=1, HV=2, K=32, V=16, has_h0=True)
    g = d["g"]
    g[0, 5, 0, :] = -30.0
    g[0, 63, 1, :] = -1000.0
    g[0, 64, 0, :] = -np.inf
    g[0, 70:90, 1, 3] = -np.inf
    g[0, 100:116, 0, :] = -11.0
    g[0, 120:137, 1, :10] = -np.inf
    g[0, 199, :, :] = -np.inf
    args = {k: d[k] for k in ("q", "k", "v", "beta")}
    o, ht = recurrent(**args, g=g, scale=d["scale"], h0=d["h0"])
    o2, ht2 = recurrent(**args, g=np.maximum(g, -10.0), scale=d["scale"], h0=d["h0"])
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    smax = max(np.abs(ht).max(), np.abs(d["h0"]).max())
    assert np.abs(o2 - o).max() < 5e-5 * smax
    assert np.abs(ht2 - ht).max() < 5e-5 * smax
