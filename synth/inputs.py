"""Seeded input recipes for the KDA chunked forward workloads.

Draw order per seed (one ``numpy.random.default_rng(seed)``): varlen lengths
(if any) -> q -> k -> v -> beta logits -> gate logits -> h0 (if any).
Everything is drawn in float64, then:

* q and k are L2-normalised over the key dimension (in float64);
* beta = sigmoid(logits), logits ~ N(0, 1);
* g = logsigmoid(logits), logits ~ N(2, 1), a natural-log per-dimension decay <= 0;
* q, k, v, g, beta are rounded to bfloat16 with round-to-nearest-even, directly
  from float64 (no intermediate float32 rounding);
* h0 = 0.1 * N(0, 1) rounded to float32, when the workload has an initial state.

Arrays are returned as float32 numpy arrays whose values are exactly
representable in bfloat16 (the oracle upcasts them exactly to float64; the GPU
side takes their top 16 bits).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    T: int            # tokens per sequence (fixed length) or total packed tokens (varlen)
    HQK: int
    HV: int
    K: int
    V: int
    has_h0: bool
    n_varlen: int = 0                 # >0: that many packed sequences, lengths drawn
    varlen_range: tuple = (64, 4097)  # numpy integers(lo, hi) -> lo <= len < hi
    meta: dict = field(default_factory=dict)


# The five workloads: the tiny single-head case, the small batched case with an
# initial state, the 8192-token 32-head prefill, the 16-sequence packed varlen
# case and the 32768-token grouped-value-head case.
CONFIGS = {
    1: Workload("kda_fwd_T256_H1_K64", 1, B=1, T=256, HQK=1, HV=1, K=64, V=64, has_h0=False),
    2: Workload("kda_fwd_B2_T2048_H4_K128", 2, B=2, T=2048, HQK=4, HV=4, K=128, V=128, has_h0=True),
    3: Workload("kda_fwd_prefill_T8192_H32_K128", 3, B=1, T=8192, HQK=32, HV=32, K=128, V=128,
                has_h0=False),
    4: Workload("kda_fwd_varlen16_H16_K128", 4, B=1, T=-1, HQK=16, HV=16, K=128, V=128,
                has_h0=True, n_varlen=16),
    5: Workload("kda_fwd_gva_T32768_HQK16_HV32_K128", 5, B=1, T=32768, HQK=16, HV=32, K=128,
                V=128, has_h0=False),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); returns float64.

    bfloat16 keeps 7 explicit mantissa bits, float64 has 52, so the low 45 bits of
    the float64 pattern are dropped with round-half-to-even: add 2**44 - 1 plus the
    lowest kept bit, then clear the dropped bits.  A carry out of the mantissa
    correctly bumps the exponent.  Valid for normal bfloat16 magnitudes (all
    inputs here are far from the bfloat16 overflow and underflow limits).
    """
    bits = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    bits = (bits + (np.uint64((1 << 44) - 1) + lsb)) & ~np.uint64((1 << 45) - 1)
    return bits.view(np.float64)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns of float32/float64 values that are bf16-exact."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = f.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("values are not exactly representable in bfloat16")
    return (bits >> 16).astype(np.uint16)


def _l2norm(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    # log(sigmoid(x)) = -log1p(exp(-x)), written stably for both signs
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def make_inputs(seed: int, B: int, T: int, HQK: int, HV: int, K: int, V: int,
                has_h0: bool, lengths=None, n_varlen: int = 0,
                varlen_range=(64, 4097), g_mean: float = 2.0) -> dict:
    """Draw one seeded input set.

    Fixed length: ``lengths is None and n_varlen == 0``; tensors are [B, T, H, D].
    Varlen: either ``lengths`` (explicit) or ``n_varlen`` (drawn from the rng
    first); sequences are packed into B=1, T=sum(lengths), ``cu_seqlens`` int64.
    """
    rng = np.random.default_rng(seed)
    cu = None
    if n_varlen:
        lengths = rng.integers(varlen_range[0], varlen_range[1], size=n_varlen)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        B, T = 1, int(lengths.sum())
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = B if cu is None else len(cu) - 1
    q = _l2norm(rng.standard_normal((B, T, HQK, K)))
    k = _l2norm(rng.standard_normal((B, T, HQK, K)))
    v = rng.standard_normal((B, T, HV, V))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, HV))))
    g = _logsigmoid(rng.normal(g_mean, 1.0, size=(B, T, HV, K)))
    h0 = (0.1 * rng.standard_normal((N, HV, K, V))).astype(np.float32) if has_h0 else None
    out = dict(
        q=round_to_bf16(q).astype(np.float32),
        k=round_to_bf16(k).astype(np.float32),
        v=round_to_bf16(v).astype(np.float32),
        g=round_to_bf16(g).astype(np.float32),
        beta=round_to_bf16(beta).astype(np.float32),
        h0=h0,
        cu_seqlens=cu,
        scale=1.0 / math.sqrt(K),
        B=B, T=T, HQK=HQK, HV=HV, K=K, V=V, N=N,
    )
    return out


def make_config_inputs(cfg_id: int) -> dict:
    w = CONFIGS[cfg_id]
    d = make_inputs(w.seed, w.B, w.T, w.HQK, w.HV, w.K, w.V, w.has_h0,
                    n_varlen=w.n_varlen, varlen_range=w.varlen_range)
    d["name"] = w.name
    return d


def make_grads(d: dict, seed: int, has_dht: bool = True) -> dict:
    """Seeded gradients for a backward pass over the inputs ``d`` (own rng, so the
    forward inputs are unchanged): do ~ N(0, 1) rounded to bfloat16, shaped like v;
    dht ~ 0.1 N(0, 1) rounded to float32, shaped like h0 ([N, HV, K, V]), or None."""
    rng = np.random.default_rng(seed)
    do = round_to_bf16(rng.standard_normal(np.shape(d["v"]))).astype(np.float32)
    dht = None
    if has_dht:
        dht = (0.1 * rng.standard_normal((d["N"], d["HV"], d["K"], d["V"]))).astype(np.float32)
    return dict(do=do, dht=dht)
