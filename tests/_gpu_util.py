"""Helpers for the GPU tests: seeded inputs -> device tensors, the HIP path
through the C ABI binding, and the oracle on sampled heads/sequences."""
from __future__ import annotations

import numpy as np

from oracle import recurrent

FIELDS = ("q", "k", "v", "g", "beta")


def nerr(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / den) if den > 0 else float(np.abs(a).max())


def to_device(d, device="cuda"):
    import torch
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).to(torch.bfloat16).to(device) for k in FIELDS}
    t["h0"] = None if d.get("h0") is None else torch.from_numpy(np.ascontiguousarray(d["h0"])).to(device)
    t["cu_seqlens"] = None if d.get("cu_seqlens") is None else \
        torch.from_numpy(np.asarray(d["cu_seqlens"], dtype=np.int64)).to(device)
    return t


def run_hip(d, dev=None, output_final_state=True, h0="from_inputs", workspace=None, o=None, nan_fill=True):
    """Run kda_fwd on the inputs dict d; returns (o, ht) as float64 numpy.  With
    ``nan_fill`` the outputs start as NaN, so that an element the kernels never write
    cannot pass as a finite leftover."""
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    t = dev if dev is not None else to_device(d)
    h = t["h0"] if h0 == "from_inputs" else h0
    ht = None
    if nan_fill:
        if o is None:
            o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device=t["v"].device)
        if output_final_state:
            N = t["q"].shape[0] if t["cu_seqlens"] is None else t["cu_seqlens"].numel() - 1
            ht = torch.full((N, t["v"].shape[2], t["q"].shape[3], t["v"].shape[3]), float("nan"),
                            dtype=torch.float32, device=t["v"].device)
    o_t, ht_t = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=h,
                        cu_seqlens=t["cu_seqlens"], output_final_state=output_final_state,
                        workspace=workspace, o=o, ht=ht)
    torch.cuda.synchronize()
    o_np = o_t.float().cpu().numpy().astype(np.float64)
    ht_np = None if ht_t is None else ht_t.cpu().numpy().astype(np.float64)
    return o_np, ht_np


def oracle_head(d, hv, seq=None):
    """O1 for one value head (and one sequence when varlen): returns (o [T_seq, V], ht [K, V])."""
    HV, HQK = d["HV"], d["HQK"]
    hq = hv // (HV // HQK)
    if d.get("cu_seqlens") is None:
        b = 0 if seq is None else seq
        sl = slice(None)
        h0 = None if d.get("h0") is None else d["h0"][b:b + 1, hv:hv + 1]
    else:
        cu = d["cu_seqlens"]
        b = 0
        sl = slice(int(cu[seq]), int(cu[seq + 1]))
        h0 = None if d.get("h0") is None else d["h0"][seq:seq + 1, hv:hv + 1]
    a = dict(q=d["q"][b:b + 1, sl, hq:hq + 1], k=d["k"][b:b + 1, sl, hq:hq + 1],
             v=d["v"][b:b + 1, sl, hv:hv + 1], g=d["g"][b:b + 1, sl, hv:hv + 1],
             beta=d["beta"][b:b + 1, sl, hv:hv + 1])
    o, ht = recurrent(**a, scale=d["scale"], h0=h0)
    return o[0, :, 0], ht[0, 0]
