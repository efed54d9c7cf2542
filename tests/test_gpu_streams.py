"""Calls that overlap on the GPU: the library keeps every piece of per-call state in the
caller's workspace, so calls on different streams (default priority) and from different
host threads, each with its own workspace and outputs, must give exactly the results
they give one at a time.  Compared bit for bit."""
import threading

import numpy as np
import pytest

from synth.inputs import make_grads, make_inputs

from _gpu_util import to_device
from test_gpu_bwd import scan_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


def fwd_args(d, t, stream):
    import torch
    from gated_delta_rule_chunked_amd import alloc_workspace, make_args
    o = torch.empty_like(t["v"])
    N = d["B"] if d["cu_seqlens"] is None else len(d["cu_seqlens"]) - 1
    ht = torch.empty((N, d["HV"], d["K"], d["V"]), dtype=torch.float32, device="cuda")
    a = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], t["h0"], t["cu_seqlens"], o, ht,
                  stream=stream.cuda_stream)
    ws = alloc_workspace(a, "cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    return a, (o, ht, ws)


def inputs():
    return [make_inputs(950, B=1, T=64 * 6 + 7, HQK=2, HV=4, K=128, V=64, has_h0=True),
            make_inputs(951, B=1, T=0, HQK=1, HV=2, K=64, V=32, has_h0=True, lengths=[200, 0, 65, 3]),
            make_inputs(952, B=2, T=64 * 9, HQK=1, HV=2, K=128, V=128, has_h0=False)]


def test_forward_calls_overlapping_on_separate_streams():
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd_raw
    ds = inputs()
    ts = [to_device(d) for d in ds]
    streams = [torch.cuda.Stream() for _ in ds]
    # one at a time
    ref = []
    for d, t, s in zip(ds, ts, streams):
        a, keep = fwd_args(d, t, s)
        kda_fwd_raw(a)
        torch.cuda.synchronize()
        ref.append([x.clone() for x in keep[:2]])
    # all enqueued before any waits, three rounds
    for _ in range(3):
        calls = [fwd_args(d, t, s) for d, t, s in zip(ds, ts, streams)]
        for a, _keep in calls:
            kda_fwd_raw(a)
        torch.cuda.synchronize()
        for (a, keep), r in zip(calls, ref):
            assert torch.equal(keep[0], r[0]) and torch.equal(keep[1], r[1])


def test_forward_calls_from_several_host_threads():
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd_raw
    ds = inputs()
    ts = [to_device(d) for d in ds]
    streams = [torch.cuda.Stream() for _ in ds]
    ref = []
    for d, t, s in zip(ds, ts, streams):
        a, keep = fwd_args(d, t, s)
        kda_fwd_raw(a)
        torch.cuda.synchronize()
        ref.append([x.clone() for x in keep[:2]])
    calls = [[fwd_args(d, t, s) for _ in range(4)] for d, t, s in zip(ds, ts, streams)]
    errors = []

    def work(i):
        try:
            for a, _keep in calls[i]:
                kda_fwd_raw(a)
        except Exception as e:   # surfaced below
            errors.append(e)
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(ds))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, r in enumerate(ref):
        for _a, keep in calls[i]:
            assert torch.equal(keep[0], r[0]) and torch.equal(keep[1], r[1])


def test_backward_and_forward_overlapping_on_separate_streams():
    import torch
    from gated_delta_rule_chunked_amd import (KDA_FLAG_CKPT_BF16, kda_bwd_dhu_raw, kda_bwd_dhu_workspace_bytes,
                                              kda_fwd_raw, make_bwd_args, max_chunks)
    d = make_inputs(953, B=1, T=64 * 5 + 30, HQK=1, HV=2, K=128, V=64, has_h0=False)
    gr = make_grads(d, 9530)
    x = scan_inputs(d, gr)
    bf = torch.bfloat16

    def dev(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    ins = (dev(x["qg"], bf), dev(x["kg"], bf), dev(x["w"], bf), dev(x["g2"], torch.float32),
           dev(x["do"], bf), dev(x["dv"], bf), dev(x["dht"], torch.float32))
    B, T, HV, K, V, N = d["B"], d["T"], d["HV"], d["K"], d["V"], d["B"]
    C = max_chunks(T, N, B, False)
    s_b, s_f = torch.cuda.Stream(), torch.cuda.Stream()

    def bwd_call(seg):
        outs = (torch.empty((B, T, HV, V), dtype=bf, device="cuda"),
                torch.empty((N, HV, K, V), dtype=torch.float32, device="cuda"),
                torch.empty((C, HV, K, V), dtype=bf, device="cuda"))
        a = make_bwd_args(*ins, d["scale"], None, *outs, stream=s_b.cuda_stream, flags=KDA_FLAG_CKPT_BF16,
                          seg_chunks=seg)
        ws = torch.empty(max(kda_bwd_dhu_workspace_bytes(a), 256), dtype=torch.uint8, device="cuda")
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        return a, outs, ws

    fd = inputs()[0]
    ft = to_device(fd)
    ref_b = []
    for seg in (0, 2):
        a, outs, _ws = bwd_call(seg)
        kda_bwd_dhu_raw(a)
        torch.cuda.synchronize()
        ref_b.append([o.clone() for o in outs])
    fa, fkeep = fwd_args(fd, ft, s_f)
    kda_fwd_raw(fa)
    torch.cuda.synchronize()
    ref_f = [o.clone() for o in fkeep[:2]]
    for _ in range(3):
        calls = [bwd_call(0), bwd_call(2)]
        fa, fkeep = fwd_args(fd, ft, s_f)
        kda_bwd_dhu_raw(calls[0][0])
        kda_fwd_raw(fa)
        kda_bwd_dhu_raw(calls[1][0])
        torch.cuda.synchronize()
        for (a, outs, _ws), r in zip(calls, ref_b):
            assert all(torch.equal(o, q) for o, q in zip(outs, r))
        assert torch.equal(fkeep[0], ref_f[0]) and torch.equal(fkeep[1], ref_f[1])


def test_library_loaded_before_torch_shares_its_runtime():
    # a fresh process that loads the library before importing torch itself: the binding
    # imports torch first, so both use one HIP runtime and a call on torch tensors works
    import os
    import subprocess
    import sys
    code = ("import gated_delta_rule_chunked_amd as pkg\n"
            "pkg.load_library()\n"
            "import torch\n"
            "from synth.inputs import make_inputs\n"
            "d = make_inputs(5, B=1, T=100, HQK=1, HV=2, K=64, V=32, has_h0=False)\n"
            "t = {k: torch.from_numpy(d[k]).to(torch.bfloat16).cuda() for k in ('q', 'k', 'v', 'g', 'beta')}\n"
            "o, ht = pkg.kda_fwd(t['q'], t['k'], t['v'], t['g'], t['beta'], scale=d['scale'])\n"
            "torch.cuda.synchronize()\n"
            "print('ok', bool(torch.isfinite(o.float()).all()))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok True" in r.stdout
