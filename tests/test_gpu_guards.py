"""No write outside the outputs, through the C ABI: every output (o, ht, hc of the forward;
dv2, dh0, dhc of the backward) is a view into a larger buffer whose margins before and
after it hold a sentinel bit pattern.  After the call the margins must be unchanged and
the outputs must equal those of a plain call bit for bit; ragged tails, varlen with
empty and one-token sequences, forced segments and chunk 16 included."""
import numpy as np
import pytest

from synth.inputs import make_grads, make_inputs

from _gpu_util import to_device
from test_gpu_bwd import scan_inputs

pytestmark = pytest.mark.gpu
GUARD = 4096        # elements of margin on each side (8 or 16 KiB: keeps every view 256-byte aligned)
SENTINEL = 0x7B3D   # a finite bf16 bit pattern (half of an fp32 word in the fp32 buffers)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


def guarded(shape, dtype):
    """A tensor of `shape` inside a buffer with sentinel margins: (view, buffer)."""
    import torch
    n = int(np.prod(shape))
    buf = torch.empty(n + 2 * GUARD, dtype=dtype, device="cuda")
    buf.view(torch.int16 if buf.element_size() == 2 else torch.int32).fill_(
        SENTINEL if buf.element_size() == 2 else (SENTINEL << 16) | SENTINEL)
    return buf[GUARD:GUARD + n].view(*shape), buf


def margins_intact(buf):
    import torch
    raw = buf.view(torch.int16 if buf.element_size() == 2 else torch.int32).cpu().numpy()
    want = SENTINEL if buf.element_size() == 2 else (SENTINEL << 16) | SENTINEL
    return np.all(raw[:GUARD] == np.array(want, raw.dtype)) and np.all(raw[-GUARD:] == np.array(want, raw.dtype))


FWD_CASES = {
    "ragged": (dict(B=2, T=64 * 3 + 17, HQK=1, HV=2, K=128, V=64), None, {}),
    "varlen": (dict(B=1, T=0, HQK=2, HV=4, K=128, V=48), [70, 0, 129, 1, 64], {}),
    "seg1": (dict(B=1, T=64 * 4 + 5, HQK=1, HV=2, K=64, V=32), None, {"seg_chunks": 1}),
    "chunk16": (dict(B=2, T=64 * 2 + 9, HQK=1, HV=2, K=128, V=64), None, {"chunk": 16}),
}


@pytest.mark.parametrize("case", list(FWD_CASES))
def test_forward_writes_nothing_outside_its_outputs(case):
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd, max_chunks
    shape, lengths, opts = FWD_CASES[case]
    d = make_inputs(900 + len(case), has_h0=True, lengths=lengths, **shape)
    t = to_device(d)
    B, T, HV, K, V = d["B"], d["T"], d["HV"], d["K"], d["V"]
    N = B if d["cu_seqlens"] is None else len(d["cu_seqlens"]) - 1
    chunk_states = opts.get("chunk", 64) == 64
    o, ob = guarded((B, T, HV, V), torch.bfloat16)
    ht, hb = guarded((N, HV, K, V), torch.float32)
    hc, cb = (guarded((max_chunks(T, N, B, d["cu_seqlens"] is not None), HV, K, V), torch.float32)
              if chunk_states else (None, None))
    kw = dict(scale=d["scale"], h0=t["h0"], cu_seqlens=t["cu_seqlens"], **opts)
    out = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], o=o, ht=ht, hc=hc,
                  output_chunk_states=chunk_states, **kw)
    plain = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], output_chunk_states=chunk_states, **kw)
    torch.cuda.synchronize()
    assert margins_intact(ob) and margins_intact(hb)
    assert torch.equal(out[0], plain[0]) and torch.equal(out[1], plain[1])
    if chunk_states:
        assert margins_intact(cb)
        n_written = (B * ((T + 63) // 64) if d["cu_seqlens"] is None else
                     int(sum((b - a + 63) // 64 for a, b in zip(d["cu_seqlens"][:-1], d["cu_seqlens"][1:]))))
        assert torch.equal(out[2][:n_written], plain[2][:n_written])


@pytest.mark.parametrize("case", ["ragged", "varlen", "seg2"])
def test_backward_writes_nothing_outside_its_outputs(case):
    import torch
    from gated_delta_rule_chunked_amd import KDA_FLAG_CKPT_BF16, kda_bwd_dhu_raw, kda_bwd_dhu_workspace_bytes
    from gated_delta_rule_chunked_amd import make_bwd_args, max_chunks
    if case == "varlen":
        d = make_inputs(930, B=1, T=0, HQK=1, HV=2, K=128, V=64, has_h0=False, lengths=[130, 0, 1, 200])
    else:
        d = make_inputs(931, B=2, T=64 * 4 + 21, HQK=1, HV=2, K=128, V=64, has_h0=False)
    gr = make_grads(d, 9300)
    x = scan_inputs(d, gr)
    B, T, HV, K, V = d["B"], d["T"], d["HV"], d["K"], d["V"]
    N = B if d["cu_seqlens"] is None else len(d["cu_seqlens"]) - 1
    C = max_chunks(T, N, B, d["cu_seqlens"] is not None)
    bf = torch.bfloat16

    def dev(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    ins = (dev(x["qg"], bf), dev(x["kg"], bf), dev(x["w"], bf), dev(x["g2"], torch.float32),
           dev(x["do"], bf), dev(x["dv"], bf), dev(x["dht"], torch.float32))
    cu = None if d["cu_seqlens"] is None else torch.from_numpy(np.asarray(d["cu_seqlens"], np.int64)).cuda()
    seg = 2 if case == "seg2" else 0

    def call(dv2, dh0, dhc):
        a = make_bwd_args(*ins, d["scale"], cu, dv2, dh0, dhc, flags=KDA_FLAG_CKPT_BF16, seg_chunks=seg)
        ws = torch.empty(max(kda_bwd_dhu_workspace_bytes(a), 256), dtype=torch.uint8, device="cuda")
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        kda_bwd_dhu_raw(a)
        torch.cuda.synchronize()

    dv2, vb = guarded((B, T, HV, V), bf)
    dh0, hb = guarded((N, HV, K, V), torch.float32)
    dhc, cb = guarded((C, HV, K, V), bf)
    call(dv2, dh0, dhc)
    p_dv2 = torch.empty((B, T, HV, V), dtype=bf, device="cuda")
    p_dh0 = torch.empty((N, HV, K, V), dtype=torch.float32, device="cuda")
    p_dhc = torch.empty((C, HV, K, V), dtype=bf, device="cuda")
    call(p_dv2, p_dh0, p_dhc)
    assert margins_intact(vb) and margins_intact(hb) and margins_intact(cb)
    n_written = (B * ((T + 63) // 64) if d["cu_seqlens"] is None else
                 int(sum((b - a + 63) // 64 for a, b in zip(d["cu_seqlens"][:-1], d["cu_seqlens"][1:]))))
    assert torch.equal(dv2, p_dv2) and torch.equal(dh0, p_dh0) and torch.equal(dhc[:n_written], p_dhc[:n_written])
