"""The calls under HIP graph capture: every kernel a call launches goes onto the caller's
stream and the work counter and chunk tables are reset by kernels, not memsets, so a
captured call can be replayed.  Each graph is replayed several times, with new input
contents copied in between and the program's own eager calls and synchronisations
around the replays, and every replay must equal an eager call on the same inputs bit
for bit (the forward at fixed length and varlen, the entry point that allocates
nothing, and the backward scan)."""
import numpy as np
import pytest

from synth.inputs import make_grads, make_inputs

from _gpu_util import FIELDS, to_device
from test_gpu_bwd import scan_inputs

pytestmark = pytest.mark.gpu
REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


def _fwd_setup(d, no_alloc=False):
    import torch
    from gated_delta_rule_chunked_amd import alloc_workspace, make_args
    t = to_device(d)
    N = d["B"] if d["cu_seqlens"] is None else len(d["cu_seqlens"]) - 1
    o = torch.empty_like(t["v"])
    ht = torch.empty((N, d["HV"], d["K"], d["V"]), dtype=torch.float32, device="cuda")
    a = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], t["h0"], t["cu_seqlens"], o, ht)
    ws = None
    if not no_alloc:
        ws = alloc_workspace(a, "cuda")
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    return t, a, o, ht, ws


def _eager_fwd(d2):
    """Eager kda_fwd on inputs d2 (fresh buffers): (o, ht)."""
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    t2 = to_device(d2)
    o, ht = kda_fwd(*(t2[k] for k in FIELDS), scale=d2["scale"], h0=t2["h0"], cu_seqlens=t2["cu_seqlens"])
    torch.cuda.synchronize()
    return o, ht


@pytest.mark.parametrize("case", ["fixed_segmented", "varlen", "no_alloc"])
def test_forward_graph_replays(case):
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd_no_alloc_raw, kda_fwd_raw
    if case == "varlen":
        mk = lambda s: make_inputs(s, B=1, T=0, HQK=1, HV=2, K=128, V=64, has_h0=True, lengths=[130, 0, 64, 257, 3])
    elif case == "no_alloc":
        mk = lambda s: make_inputs(s, B=1, T=64 * 6 + 5, HQK=1, HV=2, K=128, V=64, has_h0=True)
    else:
        mk = lambda s: make_inputs(s, B=1, T=64 * 40 + 9, HQK=1, HV=2, K=128, V=128, has_h0=True)
    d = mk(960)
    t, a, o, ht, ws = _fwd_setup(d, no_alloc=case == "no_alloc")
    run = kda_fwd_no_alloc_raw if case == "no_alloc" else kda_fwd_raw
    run(a)                          # eager first call (the no-alloc scratch address is looked up here)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        a.stream = torch.cuda.current_stream().cuda_stream
        run(a)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        dr = mk(961 + r)            # new contents, same shapes and lengths
        tr = to_device(dr)
        for k in FIELDS:
            t[k].copy_(tr[k])
        t["h0"].copy_(tr["h0"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, ht_ref = _eager_fwd(dr)   # eager work between the replays
        assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref), f"replay {r}"


def test_backward_graph_replays():
    import torch
    from gated_delta_rule_chunked_amd import (KDA_FLAG_CKPT_BF16, kda_bwd_dhu, kda_bwd_dhu_raw,
                                              kda_bwd_dhu_workspace_bytes, make_bwd_args, max_chunks)
    bf = torch.bfloat16

    def dev(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()

    def staged(seed):
        d = make_inputs(seed, B=1, T=64 * 12 + 17, HQK=1, HV=2, K=128, V=64, has_h0=False)
        x = scan_inputs(d, make_grads(d, 10 * seed))
        return d, [dev(x["qg"], bf), dev(x["kg"], bf), dev(x["w"], bf), dev(x["g2"], torch.float32),
                   dev(x["do"], bf), dev(x["dv"], bf), dev(x["dht"], torch.float32)]
    d, ins = staged(970)
    B, T, HV, K, V, N = d["B"], d["T"], d["HV"], d["K"], d["V"], d["B"]
    outs = (torch.empty((B, T, HV, V), dtype=bf, device="cuda"),
            torch.empty((N, HV, K, V), dtype=torch.float32, device="cuda"),
            torch.empty((max_chunks(T, N, B, False), HV, K, V), dtype=bf, device="cuda"))
    a = make_bwd_args(*ins, d["scale"], None, *outs, flags=KDA_FLAG_CKPT_BF16, seg_chunks=3)
    ws = torch.empty(max(kda_bwd_dhu_workspace_bytes(a), 256), dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    kda_bwd_dhu_raw(a)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        a.stream = torch.cuda.current_stream().cuda_stream
        kda_bwd_dhu_raw(a)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        dr, insr = staged(971 + r)
        for dst, src in zip(ins, insr):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = kda_bwd_dhu(*insr, scale=dr["scale"], checkpoint_dtype=bf, seg_chunks=3)
        torch.cuda.synchronize()
        # kda_bwd_dhu returns (dv2, dhc, dh0); the raw call's buffers are (dv2, dh0, dhc)
        assert torch.equal(outs[0], ref[0]) and torch.equal(outs[1], ref[2]) and torch.equal(outs[2], ref[1]), \
            f"replay {r}"
