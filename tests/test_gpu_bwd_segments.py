"""The backward reverse state scan on its segmented 64-column path (kda_bwd_scan.hip),
forced with seg_chunks: sequences are cut into segments of that many chunks, a state
pass computes each segment's hand-on dh (b) and transition (M), and the full pass
starts every segment from the dh its newer neighbours hand it.  Compared with the
fp64 oracle's bwd_dhu on the kernel's own rounded inputs, as tests/test_gpu_bwd.py
does; bar max|x - x_ref| / max|x_ref| <= 1e-2 for dv2, dhc and dh0."""
import numpy as np
import pytest

from synth.inputs import make_grads, make_inputs, round_to_bf16

from test_gpu_bwd import check, reference, run_gpu, scan_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_chunked_amd import load_library
    load_library()


@pytest.mark.parametrize("seg", [1, 2, 3, 100])
@pytest.mark.parametrize("B,T,HQK,HV,K,V", [
    (2, 64 * 7 + 17, 1, 2, 128, 64),     # ragged tail, one 64-column group
    (1, 64 * 6, 1, 1, 64, 128),          # K = 64, two column groups
    (1, 64 * 5 + 3, 2, 4, 128, 80),      # grouped heads, a partial column group (V = 80)
    (1, 64 * 4, 1, 2, 128, 16),          # one active column wave
])
def test_bwd_segments_fixed_length(seg, B, T, HQK, HV, K, V):
    d = make_inputs(91, B=B, T=T, HQK=HQK, HV=HV, K=K, V=V, has_h0=False)
    gr = make_grads(d, 910)
    x = scan_inputs(d, gr)
    check(run_gpu(x, d, seg_chunks=seg), reference(x, d), f"seg {seg} B{B} T{T} HV{HV} K{K} V{V}")


@pytest.mark.parametrize("seg", [1, 2, 50])
def test_bwd_segments_varlen_with_empty_and_ragged_sequences(seg):
    d = make_inputs(92, B=1, T=0, HQK=1, HV=2, K=128, V=64, has_h0=True, lengths=[300, 0, 64, 1, 450, 0, 129])
    gr = make_grads(d, 920)
    x = scan_inputs(d, gr)
    got, ref = run_gpu(x, d, seg_chunks=seg), reference(x, d)
    check(got, ref, f"varlen seg {seg}")
    for n in (1, 5):   # empty sequences: dh0 = dht exactly
        assert np.array_equal(got[2][n], gr["dht"][n].astype(np.float64))


def test_bwd_segments_bf16_state_and_checkpoints():
    import torch
    d = make_inputs(93, B=2, T=64 * 5 + 40, HQK=2, HV=2, K=64, V=48, has_h0=False)
    gr = make_grads(d, 930)
    gr["dht"] = round_to_bf16(gr["dht"])
    x = scan_inputs(d, gr)
    ref = reference(x, d)
    got = run_gpu(x, d, state_dtype=torch.bfloat16, checkpoint_dtype=torch.bfloat16, seg_chunks=2)
    check(got, ref, "bf16, seg 2")
    got32 = run_gpu(x, d, seg_chunks=2)
    assert np.array_equal(got[1], round_to_bf16(got32[1]))    # the bf16 checkpoint is the fp32 one rounded
    assert np.array_equal(got[0], got32[0])


def test_bwd_segments_zero_dv_no_dht_and_skipped_outputs():
    d = make_inputs(94, B=1, T=64 * 9, HQK=1, HV=1, K=128, V=32, has_h0=False)
    gr = make_grads(d, 940, has_dht=False)
    x = scan_inputs(d, gr, zero_dv=True)
    ref = reference(x, d)
    check(run_gpu(x, d, seg_chunks=3), ref, "dv = 0, dht = 0, seg 3")
    dv2, dhc, dh0 = run_gpu(x, d, output_dh0=False, output_checkpoints=False, seg_chunks=3)
    assert dhc is None and dh0 is None
    from _gpu_util import nerr
    assert nerr(dv2, ref[0]) <= 1e-2


def test_bwd_segments_agree_with_the_serial_scan():
    # same inputs, serial 16-column scan (one segment would also be the 64-column path, so
    # the serial one is reached through the library's own choice at this small shape)
    d = make_inputs(95, B=1, T=64 * 3 + 5, HQK=1, HV=2, K=128, V=64, has_h0=False)
    gr = make_grads(d, 950)
    x = scan_inputs(d, gr)
    a, b = run_gpu(x, d), run_gpu(x, d, seg_chunks=1)
    from _gpu_util import nerr
    for u, v in zip(a, b):
        assert nerr(u, v) <= 5e-3


def test_bwd_long_sequence_library_plan():
    # 513 chunks, 2 value heads, the library's own choice: eight segments of 65 chunks
    # (the forward's rule), so the oldest segment's prologue hops over six inner segments
    d = make_inputs(96, B=1, T=64 * 512 + 37, HQK=1, HV=2, K=128, V=128, has_h0=False)
    gr = make_grads(d, 960)
    x = scan_inputs(d, gr)
    check(run_gpu(x, d), reference(x, d), "513 chunks, library plan")


@pytest.mark.parametrize("n_seq", [300, 2048, 2049])
def test_bwd_many_sequences_library_plan(n_seq):
    # many short varlen sequences: the library gives each (sequence, head, 64-column group)
    # its own workgroup, longest first (the chunk table kernel sorts up to 2,048 sequences
    # on the device; past that the given order); empty sequences give dh0 = dht exactly
    rng = np.random.default_rng(970 + n_seq)
    lengths = [int(x) for x in rng.integers(0, 100 if n_seq == 300 else 4, size=n_seq)]
    lengths[7] = 0
    d = make_inputs(97, B=1, T=0, HQK=1, HV=1, K=64, V=64, has_h0=False, lengths=lengths)
    gr = make_grads(d, 9700 + n_seq)
    x = scan_inputs(d, gr)
    got, ref = run_gpu(x, d), reference(x, d)
    check(got, ref, f"{n_seq} sequences")
    assert np.array_equal(got[2][7], gr["dht"][7].astype(np.float64))


@pytest.mark.parametrize("seg", [0, 2])
@pytest.mark.parametrize("K,V", [(128, 256), (64, 192), (128, 48)])
def test_bwd_wide_and_narrow_values(seg, K, V):
    # more value column groups than key column groups (V = 256 or 192: the state pass's
    # groups past K / 64 carry b columns only), and a partial group (V = 48)
    d = make_inputs(98, B=1, T=64 * 5 + 9, HQK=1, HV=2, K=K, V=V, has_h0=False)
    gr = make_grads(d, 980)
    x = scan_inputs(d, gr)
    check(run_gpu(x, d, seg_chunks=seg), reference(x, d), f"K{K} V{V} seg {seg}")
