"""Parity of the segmented state scan against the fp64 token recurrence, with the
segment length forced (kda_fwd_args.seg_chunks) so that every path runs: many
segments (the prologue chain through M and b), partial 64-column groups, K = 64,
varlen with empty and one-chunk sequences, h0 entering through the first segment,
per-chunk states and bf16 states across segment boundaries.  Bar as for the
forward: max|x - x_ref| / max|x_ref| <= 1e-2 for o, ht (and hc)."""
import numpy as np
import pytest

from oracle import chunked, recurrent
from synth.inputs import make_inputs, round_to_bf16

from _gpu_util import FIELDS, nerr, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


def run(d, t=None, **kw):
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    t = t if t is not None else to_device(d)
    out = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"],
                  cu_seqlens=t["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return [None if x is None else x.float().cpu().numpy().astype(np.float64) for x in out]


def reference(d, h0=None):
    return recurrent(**{k: d[k] for k in FIELDS}, scale=d["scale"], h0=d["h0"] if h0 is None else h0,
                     cu_seqlens=d["cu_seqlens"])


@pytest.mark.parametrize("seg", [1, 2, 3, 8])
@pytest.mark.parametrize("K,V", [(128, 64), (128, 48), (128, 80), (64, 128), (128, 256), (64, 16)])
def test_fixed_length_forced_segments(seg, K, V):
    d = make_inputs(131, B=2, T=64 * 7 + 13, HQK=2, HV=4, K=K, V=V, has_h0=True)
    o, ht = run(d, seg_chunks=seg)
    o_ref, ht_ref = reference(d)
    eo, eh = nerr(o, o_ref), nerr(ht, ht_ref)
    print(f"  seg {seg} K{K} V{V}: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert np.all(np.isfinite(o)) and eo <= TOL and eh <= TOL


@pytest.mark.parametrize("seg", [1, 2])
def test_varlen_forced_segments_with_empty_and_short_sequences(seg):
    d = make_inputs(132, B=1, T=0, HQK=1, HV=2, K=128, V=128, has_h0=True,
                    lengths=[300, 0, 64, 1, 520, 65])
    o, ht = run(d, seg_chunks=seg)
    o_ref, ht_ref = reference(d)
    eo, eh = nerr(o, o_ref), nerr(ht, ht_ref)
    print(f"  varlen seg {seg}: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert eo <= TOL and eh <= TOL
    assert np.array_equal(ht[1], d["h0"][1].astype(np.float64))     # empty sequence: ht = h0


def test_segment_length_changes_only_rounding():
    d = make_inputs(133, B=1, T=64 * 12, HQK=1, HV=2, K=128, V=64, has_h0=True)
    outs = [run(d, seg_chunks=s) for s in (1, 4, 12)]
    for o, ht in outs[1:]:
        assert nerr(o, outs[0][0]) <= 5e-3 and nerr(ht, outs[0][1]) <= 5e-3


def test_chunk_states_and_bf16_state_across_segments():
    import torch
    d = make_inputs(134, B=1, T=0, HQK=2, HV=2, K=128, V=64, has_h0=True, lengths=[257, 130, 0, 64])
    o, ht, hc = run(d, seg_chunks=2, output_chunk_states=True)
    _, _, inter = chunked(**{k: d[k] for k in FIELDS}, scale=d["scale"], h0=d["h0"],
                          cu_seqlens=d["cu_seqlens"], return_intermediates=True)
    hc_ref = np.stack([c["h"] for c in inter])
    assert hc.shape[0] >= hc_ref.shape[0]   # room for ceil(T/64) + N chunks
    hc = hc[:hc_ref.shape[0]]
    assert nerr(hc, hc_ref) <= TOL
    o_ref, ht_ref = reference(d)
    assert nerr(o, o_ref) <= TOL and nerr(ht, ht_ref) <= TOL
    # bf16 state I/O with several segments
    h0_bf = round_to_bf16(d["h0"])
    t = to_device(d)
    t["h0"] = torch.from_numpy(h0_bf).to(torch.bfloat16).cuda()
    o2, ht2 = run(d, t, seg_chunks=1, state_dtype=torch.bfloat16)
    o2_ref, ht2_ref = reference(d, h0=h0_bf)
    assert nerr(o2, o2_ref) <= TOL and nerr(ht2, ht2_ref) <= TOL
    assert np.array_equal(ht2, round_to_bf16(ht2))


def test_many_segments_long_sequence_k64():
    # 40 chunks, one chunk per segment: the prologue chain runs up to 38 products
    d = make_inputs(135, B=1, T=64 * 40, HQK=1, HV=1, K=64, V=64, has_h0=True, g_mean=4.0)
    o, ht = run(d, seg_chunks=1)
    o_ref, ht_ref = reference(d)
    eo, eh = nerr(o, o_ref), nerr(ht, ht_ref)
    print(f"  40 segments: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert eo <= TOL and eh <= TOL


def test_automatic_segmented_scan_long_sequence_few_heads():
    # 2 value heads x 8 tiles of 16 columns, 66 chunks: the library picks the
    # segmented scan (L = 9, 8 segments)
    d = make_inputs(136, B=1, T=4200, HQK=2, HV=2, K=128, V=128, has_h0=True)
    o, ht = run(d)
    o_ref, ht_ref = reference(d)
    eo, eh = nerr(o, o_ref), nerr(ht, ht_ref)
    print(f"  auto segmented: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert eo <= TOL and eh <= TOL


def test_varlen_many_sequences_longest_first_order():
    # 70 sequences x 2 heads x 2 column groups = 280 wide workgroups fill the device, so
    # the library runs one 64-column scan per sequence and hands them out longest first
    # (the chunk table kernel sorts the sequences on the device).  Every o row must be
    # written exactly by its own scan: the output starts as NaN.
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd, kda_fwd_scan_plan, make_args
    rng = np.random.default_rng(140)
    lengths = [int(x) for x in rng.integers(0, 260, size=70)]
    lengths[3], lengths[40] = 0, 1
    d = make_inputs(141, B=1, T=0, HQK=1, HV=2, K=128, V=128, has_h0=True, lengths=lengths)
    t = to_device(d)
    o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    a = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], t["h0"], t["cu_seqlens"], o, None)
    assert kda_fwd_scan_plan(a) >= max(1, -(-max(lengths) // 64))   # one segment per sequence
    out = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"],
                  cu_seqlens=t["cu_seqlens"], o=o)
    torch.cuda.synchronize()
    o_np, ht_np = [x.float().cpu().numpy().astype(np.float64) for x in out]
    assert np.all(np.isfinite(o_np))
    o_ref, ht_ref = reference(d)
    eo, eh = nerr(o_np, o_ref), nerr(ht_np, ht_ref)
    print(f"  70 sequences: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert eo <= TOL and eh <= TOL
    assert np.array_equal(ht_np[3], d["h0"][3].astype(np.float64))


def test_varlen_300_sequences_sorted_on_the_device():
    # 300 sequences (more than one workgroup's worth, so the chunk table kernel sorts
    # them with its bitonic network rather than by rank) through the 64-column scan,
    # one per sequence, longest first; every o row checked, starting from NaN
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    rng = np.random.default_rng(148)
    lengths = [int(x) for x in rng.integers(0, 150, size=300)]
    lengths[10] = 0
    d = make_inputs(149, B=1, T=0, HQK=1, HV=1, K=64, V=64, has_h0=True, lengths=lengths)
    t = to_device(d)
    o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    out = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"],
                  cu_seqlens=t["cu_seqlens"], o=o)
    torch.cuda.synchronize()
    o_np, ht_np = [x.float().cpu().numpy().astype(np.float64) for x in out]
    assert np.all(np.isfinite(o_np))
    o_ref, ht_ref = reference(d)
    eo, eh = nerr(o_np, o_ref), nerr(ht_np, ht_ref)
    print(f"  300 sequences: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert eo <= TOL and eh <= TOL
    assert np.array_equal(ht_np[10], d["h0"][10].astype(np.float64))


@pytest.mark.parametrize("n_seq", [2048, 2049])
def test_varlen_order_limit(n_seq):
    # at the limit of the device sort (2048 sequences, bitonic network over the whole
    # LDS key array) and one past it (the given order); sequences of 0 to 3 tokens
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd
    rng = np.random.default_rng(150 + n_seq)
    lengths = [int(x) for x in rng.integers(0, 4, size=n_seq)]
    d = make_inputs(151, B=1, T=0, HQK=1, HV=1, K=64, V=64, has_h0=True, lengths=lengths)
    t = to_device(d)
    o = torch.full(t["v"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    out = kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], h0=t["h0"],
                  cu_seqlens=t["cu_seqlens"], o=o)
    torch.cuda.synchronize()
    o_np, ht_np = [x.float().cpu().numpy().astype(np.float64) for x in out]
    assert np.all(np.isfinite(o_np))
    o_ref, ht_ref = reference(d)
    eo, eh = nerr(o_np, o_ref), nerr(ht_np, ht_ref)
    print(f"  {n_seq} sequences: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert eo <= TOL and eh <= TOL


def test_very_long_sequence_eight_long_segments():
    # 1,025 chunks, 2 value heads: the library picks eight segments of 129 chunks, so the
    # last segment's prologue chains seven (M, b) hops and every segment loops 129 times
    import torch
    from gated_delta_rule_chunked_amd import kda_fwd_scan_plan, make_args
    d = make_inputs(137, B=1, T=64 * 1024 + 37, HQK=1, HV=2, K=128, V=128, has_h0=True)
    t = to_device(d)
    a = make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], t["h0"], None,
                  torch.empty_like(t["v"]), None)
    plan = kda_fwd_scan_plan(a)
    assert plan == 129, plan
    o, ht = run(d, t)
    o_ref, ht_ref = reference(d)
    eo, eh = nerr(o, o_ref), nerr(ht, ht_ref)
    print(f"  1025 chunks, plan {plan}: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert np.all(np.isfinite(o)) and eo <= TOL and eh <= TOL
