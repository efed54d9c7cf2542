"""CPU oracle for the Kimi Delta Attention (KDA) chunked forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path; its inputs come from the seeded generators in ``synth/``.

Everything is float64.  Inputs are the bfloat16-rounded tensors, upcast exactly.

Sources (web pages on the KDA chunked forward):
  * "kernel-fun 0.2.0.dev1 -- kernel_fun/kda/_kernels/fwd_state.py" (a diff page
    of the kernel-fun wheel), module docstring: the intra-stage operands
    qg = q*exp2(g2), kg = k*exp2(G - g2), Aqk[i,j] = scale * q_i k_j exp2(g2_i - g2_j)
    for i >= j, and the per-chunk state scan v' = u - w h, o = scale*qg h + Aqk v',
    h <- diag(exp2(G)) h + kg^T v', with G the gate cumsum at the chunk's last row.
  * "KDA源码剖析之FlashKDA（下）" (FlashKDA source walkthrough, part 2), sections on
    phases 3-6 of the recurrence kernel: u = (v - k_decayed @ S) * beta, U = INV @ u,
    out = q_decayed @ S + Mqk @ U, S <- g_total * S + k_restored^T @ U; and the section
    on sequence information (varlen chunk table: chunks restart at each sequence start,
    tile_base = prefix count of chunks).

The per-token recurrence is not printed on any page (the blog's formula figure
was lost).  Reading taken, consistent with both pages' chunk forms:
    S_t = (I - beta_t k_t k_t^T) diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = scale * S_t^T q_t,
with g a natural-log per-dimension decay (the pages work in log2 space with exp2;
the two are the same quantity up to the factor ln 2).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, invariants, brute force and the chunk-table example the
FlashKDA page prints.  No page prints a KDA output value, so no pin compares
outputs to printed numbers.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

__all__ = ["recurrent", "chunked", "chunk_table", "sequences"]


def sequences(B: int, T: int, cu_seqlens=None):
    """(batch, bos, eos) for every sequence.

    Fixed length: sequence n is batch row n, rows [0, T).  Varlen (B == 1):
    sequence n is rows [cu[n], cu[n+1]) of the packed batch row 0
    (FlashKDA walkthrough, sequence-information section).
    """
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    if B != 1:
        raise ValueError("varlen inputs are packed into B == 1")
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def _qk_head_map(HQK: int, HV: int) -> np.ndarray:
    # value head h reads q/k head h // (HV // HQK): consecutive value heads share one
    # q/k head (a reading: the pages only use one head count)
    if HV % HQK:
        raise ValueError("HV must be a multiple of HQK")
    return np.arange(HV) // (HV // HQK)


def recurrent(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, return_states=False):
    """Token-by-token recurrence (O1), the oracle's definition of the method.

    q, k: [B, T, HQK, K]; v: [B, T, HV, V]; g: [B, T, HV, K] natural-log decay;
    beta: [B, T, HV]; h0: [N, HV, K, V] or None (zeros).
    Returns o [B, T, HV, V] and ht [N, HV, K, V] (float64); with
    ``return_states`` also the state after every token, [B, T, HV, K, V].

    Per token (decay first, then erase along k and write beta k v^T):
        S <- diag(exp g_t) S
        S <- S + beta_t k_t (v_t - S^T k_t)^T      (== (I - beta k k^T) S + beta k v^T)
        o_t = scale * S^T q_t
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, HQK, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    hq = _qk_head_map(HQK, HV)
    seqs = sequences(B, T, cu_seqlens)
    o = np.zeros((B, T, HV, V))
    ht = np.zeros((len(seqs), HV, K, V))
    states = np.zeros((B, T, HV, K, V)) if return_states else None
    for n, (b, bos, eos) in enumerate(seqs):
        S = np.zeros((HV, K, V)) if h0 is None else np.array(h0[n], dtype=np.float64)
        for t in range(bos, eos):
            kt = k[b, t][hq]                      # [HV, K]
            qt = q[b, t][hq]                      # [HV, K]
            S = np.exp(g[b, t])[:, :, None] * S   # diag(exp g_t) S_{t-1}
            pred = np.einsum("hkv,hk->hv", S, kt)  # S^T k_t: what the memory returns for k_t
            S = S + beta[b, t][:, None, None] * kt[:, :, None] * (v[b, t] - pred)[:, None, :]
            o[b, t] = scale * np.einsum("hkv,hk->hv", S, qt)
            if return_states:
                states[b, t] = S
        ht[n] = S
    if return_states:
        return o, ht, states
    return o, ht


def chunk_table(lengths, chunk: int):
    """Per-sequence chunk counts and the exclusive prefix of those counts.

    A sequence of length L splits into ceil(L / chunk) chunks, the last one
    possibly short; ``tile_base[n]`` is the number of chunks before sequence n
    (FlashKDA walkthrough, sequence-information section, and its store-warp
    section on tail chunks).
    """
    lengths = [int(x) for x in lengths]
    if any(x < 0 for x in lengths) or chunk < 1:
        raise ValueError("lengths must be >= 0 and chunk >= 1")
    n_tiles = [(x + chunk - 1) // chunk for x in lengths]
    tile_base, acc = [], 0
    for c in n_tiles:
        tile_base.append(acc)
        acc += c
    return tile_base, n_tiles


def chunk_lengths(length: int, chunk: int):
    """Row counts of the chunks of one sequence (last may be short)."""
    return [min(chunk, length - s) for s in range(0, length, chunk)]


def _chunk_intermediates(qc, kc, vc, gc, bc, scale):
    """Intra-chunk stage for one chunk of L rows, all value heads at once.

    qc, kc: [L, HV, K] (already mapped to value heads); vc: [L, HV, V];
    gc: [L, HV, K]; bc: [L, HV].  Natural-log gate; exp replaces the pages' exp2
    of log2-scaled gates (the same numbers).

      Gam      = inclusive cumsum of g over the chunk's rows
      qg_i     = q_i * exp(Gam_i)                              (kernel-fun docstring)
      kg_j     = k_j * exp(Gam_last - Gam_j)                   (kernel-fun docstring)
      Aqk[i,j] = scale * sum_d q_id k_jd exp(Gam_id - Gam_jd),  j <= i, else 0
      Akk[i,j] = beta_i * sum_d k_id k_jd exp(Gam_id - Gam_jd), j <  i, else 0
      Tm       = (I + Akk)^-1       (the FlashKDA page's INV)
      w        = Tm diag(beta) (k * exp(Gam)),   u = Tm diag(beta) v

    Akk and Tm are not printed on the pages (only INV's use is); they follow
    from unrolling the recurrence inside a chunk, which is what the pins check.
    """
    L = qc.shape[0]
    Gam = np.cumsum(gc, axis=0)                                   # [L, HV, K]
    last = Gam[-1]                                                # [HV, K]
    qg = qc * np.exp(Gam)
    kg = kc * np.exp(last[None] - Gam)
    kgam = kc * np.exp(Gam)
    # exact per-element gate inside the dot product; j > i masked before exp
    diff = Gam[:, None] - Gam[None, :]                            # [i, j, HV, K]
    incl = np.tril(np.ones((L, L), dtype=bool))
    decay = np.exp(np.where(incl[:, :, None, None], diff, -np.inf))
    Aqk = scale * np.einsum("ihd,jhd,ijhd->hij", qc, kc, decay)
    Akk = np.einsum("ihd,jhd,ijhd->hij", kc, kc, decay)
    Akk = Akk * np.tril(np.ones((L, L)), -1)[None] * bc.T[:, :, None]
    HV = qc.shape[1]
    eye = np.eye(L)
    Tm = np.stack([solve_triangular(eye + Akk[h], eye, lower=True, unit_diagonal=True)
                   for h in range(HV)])                           # [HV, L, L]
    TmB = Tm * bc.T[:, None, :]                                   # Tm diag(beta)
    w = np.einsum("hij,jhd->ihd", TmB, kgam)
    u = np.einsum("hij,jhv->ihv", TmB, vc)
    return dict(G=Gam, qg=qg, kg=kg, Aqk=Aqk, Akk=Akk, Tm=Tm, w=w, u=u, gd=last)


def chunked(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, chunk: int = 64,
            return_intermediates=False):
    """Chunked form (O2): intra-chunk stage, then the serial inter-chunk scan.

    Any chunk size >= 1; chunks restart at each sequence start and the last
    chunk of a sequence may be short.  Per chunk (kernel-fun docstring):
        v' = u - w h
        o  = scale * qg h + Aqk v'
        h  = diag(exp(Gam_last)) h + kg^T v'
    With ``return_intermediates`` also returns a list of per-chunk dicts
    (keys of ``_chunk_intermediates`` plus seq, row0, rows, vp and h, the state
    before the chunk [HV, K, V] -- the per-chunk states that the chunked backward
    pass keeps).
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, HQK, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    hq = _qk_head_map(HQK, HV)
    seqs = sequences(B, T, cu_seqlens)
    o = np.zeros((B, T, HV, V))
    ht = np.zeros((len(seqs), HV, K, V))
    inter = [] if return_intermediates else None
    for n, (b, bos, eos) in enumerate(seqs):
        h = np.zeros((HV, K, V)) if h0 is None else np.array(h0[n], dtype=np.float64)
        for r0 in range(bos, eos, chunk):
            r1 = min(eos, r0 + chunk)
            qc = q[b, r0:r1][:, hq]
            kc = k[b, r0:r1][:, hq]
            ci = _chunk_intermediates(qc, kc, v[b, r0:r1], g[b, r0:r1], beta[b, r0:r1], scale)
            h_in = h
            vp = ci["u"] - np.einsum("ihd,hdv->ihv", ci["w"], h)
            o[b, r0:r1] = (scale * np.einsum("ihd,hdv->ihv", ci["qg"], h)
                           + np.einsum("hij,jhv->ihv", ci["Aqk"], vp))
            h = np.exp(ci["gd"])[:, :, None] * h + np.einsum("jhd,jhv->hdv", ci["kg"], vp)
            if return_intermediates:
                ci.update(seq=n, row0=r0, rows=r1 - r0, vp=vp, h=h_in)
                inter.append(ci)
        ht[n] = h
    if return_intermediates:
        return o, ht, inter
    return o, ht


def bwd_dhu(qg, kg, w, gcum, do, dv_in, scale, dht=None, cu_seqlens=None, chunk: int = 64):
    """Reverse state scan of the chunked backward pass (the stage the kernel-fun page
    "kernel_fun/kda/_kernels/bwd_dhu.py" documents in its module docstring), on
    plain tensors.

    qg, kg, w: [B, T, HV, K] (qg without scale, as in ``chunked``); gcum: [B, T, HV, K]
    chunk-local inclusive cumsum of the natural-log gate (the chunk's decay is
    exp(gcum) at its last row); do, dv_in: [B, T, HV, V]; dht: [N, HV, K, V] or None.
    Per sequence and value head, dh = dht (or 0), chunks newest first:
        dhc[c] = dh                               (gradient of the state after chunk c)
        dv2    = kg dh + dv_in                    [L, V]
        dh     = diag(exp(gcum_last)) dh + scale qg^T do - w^T dv2
    and dh0 = dh after the first chunk.  Returns dv2 [B, T, HV, V], dhc [C, HV, K, V]
    with chunks numbered sequence by sequence (as ``chunked``'s intermediates), and
    dh0 [N, HV, K, V].
    """
    qg, kg, w, gcum, do, dv_in = (np.asarray(x, dtype=np.float64) for x in (qg, kg, w, gcum, do, dv_in))
    B, T, HV, K = qg.shape
    V = do.shape[3]
    seqs = sequences(B, T, cu_seqlens)
    dv2 = np.zeros((B, T, HV, V))
    dh0 = np.zeros((len(seqs), HV, K, V))
    dhc = []
    for n, (b, bos, eos) in enumerate(seqs):
        dh = np.zeros((HV, K, V)) if dht is None else np.array(dht[n], dtype=np.float64)
        starts = list(range(bos, eos, chunk))
        seq_dhc = [None] * len(starts)
        for ci in range(len(starts) - 1, -1, -1):
            r0 = starts[ci]
            r1 = min(eos, r0 + chunk)
            seq_dhc[ci] = dh
            dv = np.einsum("jhd,hdv->jhv", kg[b, r0:r1], dh) + dv_in[b, r0:r1]
            dv2[b, r0:r1] = dv
            dh = (np.exp(gcum[b, r1 - 1])[:, :, None] * dh
                  + scale * np.einsum("ihd,ihv->hdv", qg[b, r0:r1], do[b, r0:r1])
                  - np.einsum("ihd,ihv->hdv", w[b, r0:r1], dv))
        dhc.extend(seq_dhc)
        dh0[n] = dh
    dhc = np.stack(dhc) if dhc else np.zeros((0, HV, K, V))
    return dv2, dhc, dh0


def stage_inputs(q, k, v, g, beta, scale, do, cu_seqlens=None, chunk: int = 64):
    """The forward's per-chunk operands laid out as the backward scan's plain
    tensors: qg, kg, w, gcum [B, T, HV, K] and the local gradient dv_in = Aqk^T do
    [B, T, HV, V] (the part of dL/dv' that does not pass through the state)."""
    q, k, v, g, beta, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, do))
    B, T, HQK, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    hq = _qk_head_map(HQK, HV)
    out = {n: np.zeros((B, T, HV, K)) for n in ("qg", "kg", "w", "gcum")}
    out["dv_in"] = np.zeros((B, T, HV, V))
    for b, bos, eos in sequences(B, T, cu_seqlens):
        for r0 in range(bos, eos, chunk):
            r1 = min(eos, r0 + chunk)
            ci = _chunk_intermediates(q[b, r0:r1][:, hq], k[b, r0:r1][:, hq], v[b, r0:r1],
                                      g[b, r0:r1], beta[b, r0:r1], scale)
            out["qg"][b, r0:r1] = ci["qg"]
            out["kg"][b, r0:r1] = ci["kg"]
            out["w"][b, r0:r1] = ci["w"]
            out["gcum"][b, r0:r1] = ci["G"]
            out["dv_in"][b, r0:r1] = np.einsum("hij,ihv->jhv", ci["Aqk"], do[b, r0:r1])
    return out


def backward_states(q, k, v, g, beta, scale, do, dht=None, cu_seqlens=None, chunk: int = 64):
    """The state part of the chunked backward for the loss <do, o> + <dht, ht>:
    dv2 = dL/dv' per token, dhc (gradient of the state after each chunk) and
    dh0 = dL/dh0, via ``stage_inputs`` then ``bwd_dhu``."""
    si = stage_inputs(q, k, v, g, beta, scale, do, cu_seqlens, chunk)
    return bwd_dhu(si["qg"], si["kg"], si["w"], si["gcum"], do, si["dv_in"], scale, dht=dht,
                   cu_seqlens=cu_seqlens, chunk=chunk)
