"""The C ABI on the host (no GPU needed): the library loads, exports every
function ``include/kda.h`` declares, sizes the workspace, and rejects bad
arguments with the documented status before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

from gated_delta_rule_chunked_amd import kda as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        from gated_delta_rule_chunked_amd.build import build
        build()
    return K.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(K.EXPORTED)


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_struct_layout_matches_header():
    # compile-free check of the ctypes mirror: pointer fields 8-aligned, size a multiple of 8
    a = K.KdaFwdArgs
    assert a.scale.offset == 40 and a.h0.offset == 48 and a.cu_seqlens.offset == 56
    assert a.B.offset == 64 and a.N.offset == 88 and a.o.offset == 96
    assert a.workspace_bytes.offset == 120 and a.stream.offset == 128
    assert a.flags.offset == 136 and a.hc.offset == 144 and a.seg_chunks.offset == 152
    assert a.chunk.offset == 156 and ctypes.sizeof(a) == 160


def args(**over):
    a = K.KdaFwdArgs()
    fake = 1 << 20          # aligned, never dereferenced: every call below fails validation
    a.q = a.k = a.v = a.g = a.beta = fake
    a.o = a.workspace = fake
    a.scale = 0.125
    a.B, a.T, a.HQK, a.HV, a.K, a.V, a.N = 1, 256, 2, 4, 128, 128, 1
    a.workspace_bytes = 0
    for k, v in over.items():
        setattr(a, k, v)
    return a


def ws(a):
    n = ctypes.c_size_t(0)
    st = K.load_library().kda_fwd_workspace_bytes(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_workspace_bytes(lib):
    # [header | records | (segmented scan: 1 KiB pad | B | M)]: records are one per
    # (chunk, value head).  With 256 compute units (no device seen): one segment per
    # sequence when N x HV x V/64 >= 256; else, for sequences of 96 chunks or more,
    # S = clamp(256 / (N x HV x V/64), 2, 8) segments; else the serial scan when
    # N x HV x V/16 >= 128 or there are fewer than 64 chunks.  The segmented scan adds
    # one B (fp32 K x V) and one M (bf16 K x K) per (segment, value head) when a
    # sequence has more than one segment.
    KV4, KK2 = 128 * 128 * 4, 128 * 128 * 2
    # T=8192, H=32, K=V=128: 128 chunks, 64 wide workgroups -> 4 segments of 32 chunks
    st, n = ws(args(B=1, T=8192, HQK=32, HV=32))
    assert st == 0 and n == 256 + 128 * 32 * 61952 + 1024 + 4 * 32 * (KV4 + KK2)
    # T=4096, H=32: 64 chunks, 256 serial workgroups -> serial scan
    st, n = ws(args(B=1, T=4096, HQK=32, HV=32))
    assert st == 0 and n == 256 + 64 * 32 * 61952
    # T=6144, H=32: 96 chunks -> 4 segments of 24 chunks
    st, n = ws(args(B=1, T=6144, HQK=32, HV=32))
    assert st == 0 and n == 256 + 96 * 32 * 61952 + 1024 + 4 * 32 * (KV4 + KK2)
    # T=8192, H=48: 96 wide workgroups -> 2 segments of 64 chunks
    st, n = ws(args(B=1, T=8192, HQK=48, HV=48))
    assert st == 0 and n == 256 + 128 * 48 * 61952 + 1024 + 2 * 48 * (KV4 + KK2)
    st, n = ws(args(B=2, T=200, HQK=1, HV=1, K=64, V=64, N=2))
    assert st == 0 and n == 256 + 2 * 4 * 37120
    # varlen: chunk table (N + 2 int32) and per-chunk info (8 bytes per chunk of the
    # ceil(T/64) + N capacity) in the header: 16 + 7 x 4 -> 48, + 21 x 8 = 216 -> 256
    # (5 x 2 x 8 = 80 serial workgroups, 16 chunks: serial scan)
    st, n = ws(args(B=1, T=1000, HQK=1, HV=2, N=5, cu_seqlens=1 << 20))
    assert st == 0 and n == 256 + (16 + 5) * 2 * 61952
    # N=70: 70 x 2 x 2 = 280 wide workgroups fill the device: one segment per sequence;
    # header 16 + 72 x 4 + 71 x 4 (segment table) + 70 x 4 (longest-first order) = 868,
    # chunk info from 872: + 86 x 8 = 1560 -> 1792
    st, n = ws(args(B=1, T=1000, HQK=1, HV=2, N=70, cu_seqlens=1 << 20))
    assert st == 0 and n == 1792 + (16 + 70) * 2 * 61952 + 1024
    # T=16384, H=2: 16 serial workgroups, 256 chunks -> segmented, L = max(8, 256/8) = 32, 8 segments
    st, n = ws(args(B=1, T=16384, HQK=2, HV=2))
    assert st == 0 and n == 256 + 256 * 2 * 61952 + 1024 + 8 * 2 * (KV4 + KK2)
    # forced segment length 32 at T=8192: 4 segments per sequence
    st, n = ws(args(B=1, T=8192, HQK=32, HV=32, seg_chunks=32))
    assert st == 0 and n == 256 + 128 * 32 * 61952 + 1024 + 4 * 32 * (KV4 + KK2)
    # forced, one segment per sequence: no B / M
    st, n = ws(args(B=1, T=8192, HQK=32, HV=32, seg_chunks=128))
    assert st == 0 and n == 256 + 128 * 32 * 61952 + 1024
    # forced varlen: header 16 + 7 x 4 (chunk table, flag) + 6 x 4 (segment table) = 68,
    # chunk info from 72: + 21 x 8 = 240 -> 256;
    # up to (16 + 5) // 2 + 5 = 15 segments
    st, n = ws(args(B=1, T=1000, HQK=1, HV=2, N=5, cu_seqlens=1 << 20, seg_chunks=2))
    assert st == 0 and n == 256 + (16 + 5) * 2 * 61952 + 1024 + 15 * 2 * (KV4 + KK2)
    st, n = ws(args(T=0))
    assert st == 0 and n == 0
    assert ws(args(seg_chunks=-1))[0] == K.KDA_ERR_INVALID_ARG


def test_scan_plan(lib):
    # the scan choice, host only (256 compute units when no device is seen)
    plan = lambda **kw: K.kda_fwd_scan_plan(args(**kw))
    assert plan(B=1, T=8192, HQK=32, HV=32) == 32                # 4 segments: the full pass in one round
    assert plan(B=1, T=8192, HQK=48, HV=48) == 64                # 2 segments
    assert plan(B=1, T=8192, HQK=16, HV=16) == 16                # 8 segments
    assert plan(B=1, T=4096, HQK=32, HV=32) == 0                 # 64 chunks, 256 serial workgroups
    assert plan(B=4, T=8192, HQK=32, HV=32, N=4) >= 128              # 256 wide workgroups: one segment each
    assert plan(B=1, T=16384, HQK=2, HV=2) == 32                 # 8 segments
    assert plan(B=1, T=8192, HQK=32, HV=32, seg_chunks=5) == 5   # forced
    assert plan(B=1, T=200, HQK=1, HV=1) == 0
    assert plan(B=2, T=2048, HQK=4, HV=4, N=2) == 4              # 32 chunks, 64 serial workgroups: 8 segments
    assert plan(B=2, T=1984, HQK=4, HV=4, N=2) == 0              # 31 chunks: serial
    n = ctypes.c_int32(0)
    assert lib.kda_fwd_scan_plan(None, ctypes.byref(n)) == K.KDA_ERR_INVALID_ARG
    assert lib.kda_fwd_scan_plan(ctypes.byref(args()), None) == K.KDA_ERR_INVALID_ARG
    assert lib.kda_fwd_scan_plan(ctypes.byref(args(K=96)), ctypes.byref(n)) == K.KDA_ERR_UNSUPPORTED


ALL = ("kda_fwd", "kda_fwd_intra", "kda_fwd_inter")
INTRA = ("kda_fwd", "kda_fwd_intra")     # entry points that read q, k, g, beta
INTER = ("kda_fwd", "kda_fwd_inter")     # entry points that read v, o, h0, ht


@pytest.mark.parametrize("over,status,entries", [
    (dict(K=96), K.KDA_ERR_UNSUPPORTED, ALL),
    (dict(V=40), K.KDA_ERR_UNSUPPORTED, ALL),
    (dict(V=0), K.KDA_ERR_UNSUPPORTED, ALL),
    (dict(HQK=3), K.KDA_ERR_INVALID_ARG, ALL),          # HV % HQK != 0
    (dict(B=0), K.KDA_ERR_INVALID_ARG, ALL),
    (dict(T=-1), K.KDA_ERR_INVALID_ARG, ALL),
    (dict(N=2), K.KDA_ERR_INVALID_ARG, ALL),            # fixed length needs N == B
    (dict(B=2, N=2, cu_seqlens=1 << 20), K.KDA_ERR_INVALID_ARG, ALL),   # varlen needs B == 1
    (dict(cu_seqlens=(1 << 20) + 4), K.KDA_ERR_INVALID_ARG, ALL),      # misaligned int64
    (dict(q=0), K.KDA_ERR_INVALID_ARG, INTRA),
    (dict(beta=(1 << 20) + 1), K.KDA_ERR_INVALID_ARG, INTRA),
    (dict(v=(1 << 20) + 8), K.KDA_ERR_INVALID_ARG, INTER),   # misaligned
    (dict(o=0), K.KDA_ERR_INVALID_ARG, INTER),
    (dict(o=(1 << 20) + 4), K.KDA_ERR_INVALID_ARG, INTER),   # o needs 8 bytes
    (dict(h0=(1 << 20) + 4), K.KDA_ERR_INVALID_ARG, INTER),
    (dict(flags=4), K.KDA_ERR_INVALID_ARG, ALL),              # unknown option bit
    (dict(hc=(1 << 20) + 8), K.KDA_ERR_INVALID_ARG, ALL),     # misaligned per-chunk states
    (dict(chunk=32), K.KDA_ERR_UNSUPPORTED, ALL),             # chunk length 64 or 16 only
    (dict(chunk=16, hc=1 << 20, workspace_bytes=1 << 40), K.KDA_ERR_UNSUPPORTED, ALL),   # no chunk states at 16
    (dict(workspace=0), K.KDA_ERR_WORKSPACE, ALL),
    (dict(workspace_bytes=1000), K.KDA_ERR_WORKSPACE, ALL),
    (dict(workspace=(1 << 20) + 128, workspace_bytes=1 << 40), K.KDA_ERR_WORKSPACE, ALL),
    (dict(scale=float("nan"), workspace_bytes=1 << 40), K.KDA_ERR_INVALID_ARG, ALL),
])
def test_validation_rejects_before_launch(lib, over, status, entries):
    a = args(**over)
    for name in entries:
        st = getattr(lib, name)(ctypes.byref(a))
        assert st == status, (name, over, st)
    assert K.kda_strerror(status)


def test_null_args_and_strerror(lib):
    assert lib.kda_fwd(None) == K.KDA_ERR_INVALID_ARG
    assert lib.kda_fwd_workspace_bytes(None, None) == K.KDA_ERR_INVALID_ARG
    assert K.kda_strerror(0) == "ok" and K.kda_strerror(12345) == "unknown status"


# ---------------------------------------------------------------- backward scan
def test_bwd_struct_layout_matches_header():
    a = K.KdaBwdDhuArgs
    assert a.g2.offset == 24 and a.dht.offset == 48 and a.scale.offset == 56 and a.cu_seqlens.offset == 64
    assert a.B.offset == 72 and a.N.offset == 92 and a.dv2.offset == 96 and a.dhc.offset == 112
    assert a.workspace_bytes.offset == 128 and a.stream.offset == 136 and a.flags.offset == 144
    assert a.seg_chunks.offset == 148 and ctypes.sizeof(a) == 152


def bwd_args(**over):
    a = K.KdaBwdDhuArgs()
    fake = 1 << 20
    a.qg = a.kg = a.w = a.g2 = a.dout = a.dv2 = fake
    a.scale = 0.125
    a.B, a.T, a.HV, a.K, a.V, a.N = 1, 256, 4, 128, 128, 1
    for k, v in over.items():
        setattr(a, k, v)
    return a


def bwd_ws(a):
    n = ctypes.c_size_t(0)
    st = K.load_library().kda_bwd_dhu_workspace_bytes(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_bwd_workspace_bytes(lib):
    # The forward's plan (256 compute units when no device is seen).  Fixed length on the
    # serial scan needs no scratch; the segmented scan adds b (fp32 K x V) and M (bf16 K x K)
    # per (segment, head) when a sequence has several segments.  Varlen holds the chunk table
    # (N + 2 int32), with the segmented scan the segment table (N + 1), and the longest-first
    # sequence order (N, when every sequence is one scan unit, up to 2048 sequences).
    KV4, KK2 = 128 * 128 * 4, 128 * 128 * 2
    # 8192 tokens, 32 heads: 4 segments of 32 chunks
    assert bwd_ws(bwd_args(B=1, T=8192, HV=32)) == (0, 4 * 32 * (KV4 + KK2))
    assert bwd_ws(bwd_args(B=1, T=8192, HV=32, seg_chunks=128)) == (0, 0)   # one segment: no b, M
    assert bwd_ws(bwd_args(B=1, T=4096, HV=32)) == (0, 0)                   # the serial scan
    assert bwd_ws(bwd_args(N=5, cu_seqlens=1 << 20)) == (0, 256)            # serial: 7 + 5 words
    # 70 sequences: 560 wide workgroups, one segment each: 72 + 71 + 70 words -> 1024
    assert bwd_ws(bwd_args(N=70, cu_seqlens=1 << 20)) == (0, 1024)
    # 3000 sequences: no longest-first order past 2048
    assert bwd_ws(bwd_args(N=3000, cu_seqlens=1 << 20)) == (0, ((3002 + 3001) * 4 + 255) // 256 * 256)
    # forced segments of 2 chunks on 4 varlen sequences: (4 + 5) // 2 + 5 = 9 segments
    st, n = bwd_ws(bwd_args(N=5, cu_seqlens=1 << 20, HV=2, seg_chunks=2))
    assert st == 0 and n == 256 + ((4 + 5) // 2 + 5) * 2 * (KV4 + KK2)
    assert bwd_ws(bwd_args(K=96))[0] == K.KDA_ERR_UNSUPPORTED
    assert bwd_ws(bwd_args(seg_chunks=-1))[0] == K.KDA_ERR_INVALID_ARG
    assert lib.kda_bwd_dhu_workspace_bytes(None, None) == K.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("over,status", [
    (dict(K=96), K.KDA_ERR_UNSUPPORTED),
    (dict(V=24), K.KDA_ERR_UNSUPPORTED),
    (dict(B=0), K.KDA_ERR_INVALID_ARG),
    (dict(N=2), K.KDA_ERR_INVALID_ARG),
    (dict(B=2, N=2, cu_seqlens=1 << 20), K.KDA_ERR_INVALID_ARG),
    (dict(qg=0), K.KDA_ERR_INVALID_ARG),
    (dict(g2=0), K.KDA_ERR_INVALID_ARG),
    (dict(dv2=0), K.KDA_ERR_INVALID_ARG),
    (dict(w=(1 << 20) + 8), K.KDA_ERR_INVALID_ARG),       # K-wide operands need 16 bytes
    (dict(dout=(1 << 20) + 4), K.KDA_ERR_INVALID_ARG),    # V-wide tensors need 8 bytes
    (dict(dhc=(1 << 20) + 8), K.KDA_ERR_INVALID_ARG),
    (dict(dht=(1 << 20) + 8), K.KDA_ERR_INVALID_ARG),
    (dict(flags=1), K.KDA_ERR_INVALID_ARG),               # the forward's beta option
    (dict(flags=8), K.KDA_ERR_INVALID_ARG),
    (dict(N=5, cu_seqlens=1 << 20), K.KDA_ERR_WORKSPACE),  # varlen needs the table
    (dict(N=5, cu_seqlens=1 << 20, workspace=1 << 20, workspace_bytes=100), K.KDA_ERR_WORKSPACE),
    (dict(scale=float("nan")), K.KDA_ERR_INVALID_ARG),
])
def test_bwd_validation_rejects_before_launch(lib, over, status):
    assert lib.kda_bwd_dhu(ctypes.byref(bwd_args(**over))) == status
    assert lib.kda_bwd_dhu(None) == K.KDA_ERR_INVALID_ARG


def test_no_alloc_rejects_shapes_beyond_its_static_buffer(lib):
    # the 8192-token, 32-head workload needs about 270 MB of workspace, more than the
    # static scratch of kda_fwd_no_alloc holds: refused before any device call
    a = args(B=1, T=8192, HQK=32, HV=32)
    st, n = ws(a)
    assert st == 0 and n > K.KDA_NO_ALLOC_MAX_BYTES
    assert lib.kda_fwd_no_alloc(ctypes.byref(a)) == K.KDA_ERR_TOO_LARGE
    assert "KDA_NO_ALLOC_MAX_BYTES" in K.kda_strerror(K.KDA_ERR_TOO_LARGE)
    assert lib.kda_fwd_no_alloc(None) == K.KDA_ERR_INVALID_ARG


def test_shape_limits(lib):
    # the largest shapes the kernels' 32-bit grid and record indices take, and one past them
    limit = (1 << 31) - 8                                     # (chunk, value head) records
    hv = 1 << 20
    st, n = ws(args(B=1, T=64 * 2047, HQK=1, HV=hv, N=1))     # 2047 * 2^20 records: inside
    assert st == 0 and n >= 2047 * hv * 61952 and 2047 * hv < limit
    assert ws(args(B=1, T=64 * 2048, HQK=1, HV=hv, N=1))[0] == K.KDA_ERR_INVALID_ARG   # 2^31 records
    assert ws(args(B=1 << 20, T=1 << 21, HQK=1, HV=1, N=1 << 20))[0] == K.KDA_ERR_INVALID_ARG  # 2^41 rows
    # varlen: at most 2^30 - 1 sequences
    assert ws(args(B=1, T=1 << 20, N=(1 << 30), cu_seqlens=1 << 20))[0] == K.KDA_ERR_INVALID_ARG
    st, n = ws(args(B=1, T=1 << 20, N=(1 << 20), cu_seqlens=1 << 20))
    assert st == 0 and n > 0
    # the backward's limits are the same
    assert bwd_ws(bwd_args(B=1, T=64 * 2048, HV=hv, N=1))[0] == K.KDA_ERR_INVALID_ARG
    assert bwd_ws(bwd_args(B=1, T=64 * 2047, HV=hv, N=1))[0] == 0
