"""Python binding of the C ABI in ``include/kda.h`` (ctypes).

Argument marshalling only: every step of the forward runs in the HIP kernels of
``libkda.so``.  PyTorch supplies device memory (outputs, workspace) and the
current stream.  There is no CPU fallback: if the library is missing or no GPU
is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_int32, c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARG = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_WORKSPACE = -3
KDA_ERR_HIP = -4
KDA_ERR_TOO_LARGE = -5
KDA_NO_ALLOC_MAX_BYTES = 128 << 20
KDA_CHUNK = 64
KDA_FLAG_BETA_LOGITS = 1
KDA_FLAG_STATE_BF16 = 2
KDA_FLAG_CKPT_BF16 = 4

EXPORTED = ("kda_fwd_workspace_bytes", "kda_fwd_scan_plan", "kda_fwd", "kda_fwd_no_alloc", "kda_fwd_intra",
            "kda_fwd_inter", "kda_debug_unpack", "kda_bwd_dhu_workspace_bytes", "kda_bwd_dhu", "kda_strerror")


class KdaFwdArgs(ctypes.Structure):
    """Mirror of ``kda_fwd_args`` (field order and types as in the header)."""
    _fields_ = [
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("g", c_void_p), ("beta", c_void_p),
        ("scale", c_float), ("h0", c_void_p), ("cu_seqlens", c_void_p),
        ("B", c_int32), ("T", c_int32), ("HQK", c_int32), ("HV", c_int32),
        ("K", c_int32), ("V", c_int32), ("N", c_int32),
        ("o", c_void_p), ("ht", c_void_p),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("stream", c_void_p),
        ("flags", ctypes.c_uint32), ("hc", c_void_p),
        ("seg_chunks", c_int32), ("chunk", c_int32),
    ]


class KdaBwdDhuArgs(ctypes.Structure):
    """Mirror of ``kda_bwd_dhu_args`` (field order and types as in the header)."""
    _fields_ = [
        ("qg", c_void_p), ("kg", c_void_p), ("w", c_void_p), ("g2", c_void_p),
        ("dout", c_void_p), ("dv", c_void_p), ("dht", c_void_p),
        ("scale", c_float), ("cu_seqlens", c_void_p),
        ("B", c_int32), ("T", c_int32), ("HV", c_int32), ("K", c_int32), ("V", c_int32), ("N", c_int32),
        ("dv2", c_void_p), ("dh0", c_void_p), ("dhc", c_void_p),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("stream", c_void_p), ("flags", ctypes.c_uint32), ("seg_chunks", c_int32),
    ]


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status}: {kda_strerror(status)}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load ``libkda.so`` once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gated_delta_rule_chunked_amd.build`")
    # torch ships its own HIP runtime; loaded first, it is the one libkda.so binds to, so
    # that the library and torch's tensors and streams share one runtime (loaded the other
    # way round, the process holds two runtimes and the library sees no device of torch's)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(KdaFwdArgs)
    lib.kda_fwd_workspace_bytes.argtypes = [P, ctypes.POINTER(c_size_t)]
    for name in ("kda_fwd", "kda_fwd_no_alloc", "kda_fwd_intra", "kda_fwd_inter"):
        getattr(lib, name).argtypes = [P]
        getattr(lib, name).restype = c_int
    lib.kda_fwd_workspace_bytes.restype = c_int
    lib.kda_fwd_scan_plan.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    lib.kda_fwd_scan_plan.restype = c_int
    lib.kda_debug_unpack.argtypes = [P] + [c_void_p] * 6
    lib.kda_debug_unpack.restype = c_int
    PB = ctypes.POINTER(KdaBwdDhuArgs)
    lib.kda_bwd_dhu_workspace_bytes.argtypes = [PB, ctypes.POINTER(c_size_t)]
    lib.kda_bwd_dhu_workspace_bytes.restype = c_int
    lib.kda_bwd_dhu.argtypes = [PB]
    lib.kda_bwd_dhu.restype = c_int
    lib.kda_strerror.argtypes = [c_int]
    lib.kda_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def kda_strerror(status: int) -> str:
    return load_library().kda_strerror(status).decode()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, shape, dtype, device, min_rows=False):
    """Exact shape (or, with ``min_rows``, at least shape[0] rows), dtype, contiguity
    and device of one argument tensor."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    ok = tuple(t.shape[1:]) == tuple(shape[1:]) and t.dim() == len(shape) and \
        (t.shape[0] >= shape[0] if min_rows else t.shape[0] == shape[0])
    if not ok:
        want = ("[>=%d, " % shape[0] + ", ".join(map(str, shape[1:])) + "]") if min_rows else list(shape)
        raise ValueError(f"{name} must have shape {want}, got {list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")


def max_chunks(T, N, B=1, varlen=False):
    """Room for the chunks of every sequence: B * ceil(T/64) for fixed length; for
    varlen (N packed sequences in T tokens) ceil(T/64) + N, an upper bound of
    sum_n ceil(len_n / 64) that needs no look at the lengths."""
    nt = (T + KDA_CHUNK - 1) // KDA_CHUNK
    return nt + N if varlen else B * nt


def make_args(q, k, v, g, beta, scale=None, h0=None, cu_seqlens=None, o=None, ht=None,
              workspace=None, stream=None, flags=0, hc=None, seg_chunks=0, chunk=64) -> KdaFwdArgs:
    """Fill ``kda_fwd_args`` from torch tensors (shapes as in the header).

    q, k: [B, T, HQK, K] bf16; v: [B, T, HV, V] bf16; g: [B, T, HV, K] bf16;
    beta: [B, T, HV] bf16; h0: [N, HV, K, V] or None; cu_seqlens: int64 [N+1]
    on the device or None; o: [B, T, HV, V] bf16; ht: [N, HV, K, V] or None;
    hc: [C, HV, K, V] or None, C = B * ceil(T/64) for fixed length and at least
    ceil(T/64) + N for varlen (see ``max_chunks``).  States (h0, ht, hc) are fp32,
    or bf16 with KDA_FLAG_STATE_BF16 in ``flags``.  Every tensor must be contiguous
    and on q's device (the C ABI sees only pointers, so this is the only check of
    the sizes it will read and write); violations raise ValueError or TypeError.
    """
    import torch
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be 4-dimensional: [B, T, HQK, K] and [B, T, HV, V]")
    B, T, HQK, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dev = q.device
    if cu_seqlens is not None and (cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2):
        raise ValueError("cu_seqlens must be a 1-dimensional int64 tensor of N + 1 >= 2 offsets")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    sdt = torch.bfloat16 if flags & KDA_FLAG_STATE_BF16 else torch.float32
    bf = torch.bfloat16
    C = max_chunks(T, N, B, cu_seqlens is not None)
    for name, t, shape, dt in (("q", q, (B, T, HQK, K), bf), ("k", k, (B, T, HQK, K), bf),
                               ("v", v, (B, T, HV, V), bf), ("g", g, (B, T, HV, K), bf),
                               ("beta", beta, (B, T, HV), bf), ("h0", h0, (N, HV, K, V), sdt),
                               ("cu_seqlens", cu_seqlens, (N + 1,), torch.int64),
                               ("o", o, (B, T, HV, V), bf), ("ht", ht, (N, HV, K, V), sdt)):
        _check_tensor(name, t, shape, dt, dev)
    # varlen: the exact chunk count depends on the lengths, which stay on the device
    _check_tensor("hc", hc, (C, HV, K, V), sdt, dev, min_rows=cu_seqlens is not None)
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a HIP device, they are on {dev}")
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    a = KdaFwdArgs()
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.scale = float(K ** -0.5 if scale is None else scale)
    a.h0, a.cu_seqlens = _ptr(h0), _ptr(cu_seqlens)
    a.B, a.T, a.HQK, a.HV, a.K, a.V, a.N = B, T, HQK, HV, K, V, N
    a.o, a.ht = _ptr(o), _ptr(ht)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.stream = stream
    a.flags = int(flags)
    a.hc = _ptr(hc)
    a.seg_chunks = int(seg_chunks)
    a.chunk = int(chunk)
    return a


def kda_fwd_scan_plan(args: KdaFwdArgs) -> int:
    """Segment length of the 64-column scan these arguments select, or 0 for the
    16-column serial scan (host only)."""
    n = ctypes.c_int32(0)
    st = load_library().kda_fwd_scan_plan(ctypes.byref(args), ctypes.byref(n))
    if st != KDA_OK:
        raise KdaError(st, "kda_fwd_scan_plan")
    return n.value


def kda_fwd_workspace_bytes(args: KdaFwdArgs) -> int:
    n = c_size_t(0)
    st = load_library().kda_fwd_workspace_bytes(ctypes.byref(args), ctypes.byref(n))
    if st != KDA_OK:
        raise KdaError(st, "kda_fwd_workspace_bytes")
    return n.value


def _call(name: str, args: KdaFwdArgs) -> None:
    st = getattr(load_library(), name)(ctypes.byref(args))
    if st != KDA_OK:
        raise KdaError(st, name)


def kda_fwd_raw(args: KdaFwdArgs) -> None:
    _call("kda_fwd", args)


def kda_fwd_no_alloc_raw(args: KdaFwdArgs) -> None:
    """kda_fwd on the library's static per-device scratch (``args.workspace`` is
    ignored); raises KdaError with KDA_ERR_TOO_LARGE when the shapes need more than
    KDA_NO_ALLOC_MAX_BYTES."""
    _call("kda_fwd_no_alloc", args)


def kda_fwd_intra(args: KdaFwdArgs) -> None:
    _call("kda_fwd_intra", args)


def kda_fwd_inter(args: KdaFwdArgs) -> None:
    _call("kda_fwd_inter", args)


def alloc_workspace(args: KdaFwdArgs, device):
    import torch
    n = kda_fwd_workspace_bytes(args)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def num_chunks(T, cu_seqlens=None, B=1):
    """Chunks over all sequences: B * ceil(T/64), or sum_n ceil(len_n/64) for varlen.
    For varlen this reads cu_seqlens on the host: a device tensor is copied, which
    synchronises with the device (the forward and backward calls never do this; they
    size per-chunk outputs by ``max_chunks``)."""
    if cu_seqlens is None:
        return B * ((T + KDA_CHUNK - 1) // KDA_CHUNK)
    cu = [int(x) for x in cu_seqlens.detach().cpu().tolist()]
    return sum((cu[i + 1] - cu[i] + KDA_CHUNK - 1) // KDA_CHUNK for i in range(len(cu) - 1))


def kda_fwd(q, k, v, g, beta, scale=None, h0=None, cu_seqlens=None, output_final_state=True,
            o=None, workspace=None, beta_logits=False, state_dtype=None, output_chunk_states=False,
            seg_chunks=0, ht=None, hc=None, chunk=64):
    """Chunked KDA forward on the current stream.

    Returns (o, ht or None), or (o, ht or None, hc) with ``output_chunk_states``:
    hc [C, HV, K, V] is the state before each chunk, chunks numbered sequence by
    sequence.  For fixed length C = B * ceil(T/64); for varlen hc is allocated with
    ``max_chunks`` = ceil(T/64) + N rows, of which the first sum_n ceil(len_n/64) are
    written (the lengths are not read on the host, so the call never synchronises).
    ``beta_logits``: beta holds logits and the kernel applies the sigmoid.
    ``state_dtype``: torch.float32 (default) or torch.bfloat16 for h0, ht and hc.
    ``seg_chunks``: segment length of the state scan in chunks (0: chosen by the library).
    ``chunk``: 64 (default) or 16, FlashKDA's chunk length (no chunk states with 16).
    Allocates o, ht, hc and the workspace with torch unless given.
    """
    import torch
    if not q.is_cuda:
        raise RuntimeError("kda_fwd runs on the GPU only (tensors must be on a HIP device)")
    load_library()
    with torch.cuda.device(q.device):   # the library launches on the current device
        return _kda_fwd_on_device(q, k, v, g, beta, scale, h0, cu_seqlens, output_final_state, o, workspace,
                                  beta_logits, state_dtype, output_chunk_states, seg_chunks, ht, hc, chunk)


def _kda_fwd_on_device(q, k, v, g, beta, scale, h0, cu_seqlens, output_final_state, o, workspace, beta_logits,
                       state_dtype, output_chunk_states, seg_chunks, ht, hc, chunk):
    import torch
    B, T, _, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    sdt = torch.float32 if state_dtype is None else state_dtype
    if sdt not in (torch.float32, torch.bfloat16):
        raise TypeError("state_dtype must be torch.float32 or torch.bfloat16")
    flags = (KDA_FLAG_BETA_LOGITS if beta_logits else 0) | (KDA_FLAG_STATE_BF16 if sdt == torch.bfloat16 else 0)
    if o is None:
        o = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=q.device)
    if ht is None and output_final_state:
        ht = torch.empty((N, HV, K, V), dtype=sdt, device=q.device)
    if not output_final_state:
        ht = None
    if output_chunk_states and hc is None:
        hc = torch.empty((max_chunks(T, N, B, cu_seqlens is not None), HV, K, V), dtype=sdt, device=q.device)
    if not output_chunk_states:
        hc = None
    args = make_args(q, k, v, g, beta, scale, h0, cu_seqlens, o, ht, flags=flags, hc=hc, seg_chunks=seg_chunks,
                     chunk=chunk)
    if workspace is None:
        workspace = alloc_workspace(args, q.device)
    args.workspace = workspace.data_ptr()
    args.workspace_bytes = workspace.numel() * workspace.element_size()
    kda_fwd_raw(args)
    return (o, ht, hc) if output_chunk_states else (o, ht)


def kda_debug_unpack(args: KdaFwdArgs, qg=None, w=None, kg=None, aqk=None, tmb=None, alpha=None):
    st = load_library().kda_debug_unpack(ctypes.byref(args), _ptr(qg), _ptr(w), _ptr(kg), _ptr(aqk),
                                         _ptr(tmb), _ptr(alpha))
    if st != KDA_OK:
        raise KdaError(st, "kda_debug_unpack")


def make_bwd_args(qg, kg, w, g2, do, dv=None, dht=None, scale=None, cu_seqlens=None, dv2=None, dh0=None,
                  dhc=None, workspace=None, stream=None, flags=0, seg_chunks=0) -> KdaBwdDhuArgs:
    """Fill ``kda_bwd_dhu_args`` from torch tensors (shapes as in the header).

    qg, kg, w: [B, T, HV, K] bf16; g2: [B, T, HV, K] fp32; do, dv, dv2: [B, T, HV, V]
    bf16; dht, dh0: [N, HV, K, V] fp32 (bf16 with KDA_FLAG_STATE_BF16); dhc:
    [C, HV, K, V] fp32 (bf16 with KDA_FLAG_CKPT_BF16), C as hc of ``make_args``.
    Shapes, dtypes, contiguity and the device are checked as in ``make_args``.
    """
    import torch
    if qg.dim() != 4 or do.dim() != 4:
        raise ValueError("qg and do must be 4-dimensional: [B, T, HV, K] and [B, T, HV, V]")
    B, T, HV, K = qg.shape
    V = do.shape[3]
    dev = qg.device
    if cu_seqlens is not None and (cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2):
        raise ValueError("cu_seqlens must be a 1-dimensional int64 tensor of N + 1 >= 2 offsets")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    sdt = torch.bfloat16 if flags & KDA_FLAG_STATE_BF16 else torch.float32
    cdt = torch.bfloat16 if flags & KDA_FLAG_CKPT_BF16 else torch.float32
    bf = torch.bfloat16
    C = max_chunks(T, N, B, cu_seqlens is not None)
    for name, t, shape, dt in (("qg", qg, (B, T, HV, K), bf), ("kg", kg, (B, T, HV, K), bf),
                               ("w", w, (B, T, HV, K), bf), ("g2", g2, (B, T, HV, K), torch.float32),
                               ("do", do, (B, T, HV, V), bf), ("dv", dv, (B, T, HV, V), bf),
                               ("dht", dht, (N, HV, K, V), sdt), ("cu_seqlens", cu_seqlens, (N + 1,), torch.int64),
                               ("dv2", dv2, (B, T, HV, V), bf), ("dh0", dh0, (N, HV, K, V), sdt)):
        _check_tensor(name, t, shape, dt, dev)
    _check_tensor("dhc", dhc, (C, HV, K, V), cdt, dev, min_rows=cu_seqlens is not None)
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a HIP device, they are on {dev}")
    if stream is None:
        stream = torch.cuda.current_stream(qg.device).cuda_stream
    a = KdaBwdDhuArgs()
    a.qg, a.kg, a.w, a.g2 = _ptr(qg), _ptr(kg), _ptr(w), _ptr(g2)
    a.dout, a.dv, a.dht = _ptr(do), _ptr(dv), _ptr(dht)
    a.scale = float(K ** -0.5 if scale is None else scale)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.B, a.T, a.HV, a.K, a.V, a.N = B, T, HV, K, V, N
    a.dv2, a.dh0, a.dhc = _ptr(dv2), _ptr(dh0), _ptr(dhc)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.stream = stream
    a.flags = int(flags)
    a.seg_chunks = int(seg_chunks)
    return a


def kda_bwd_dhu_workspace_bytes(args: KdaBwdDhuArgs) -> int:
    n = c_size_t(0)
    st = load_library().kda_bwd_dhu_workspace_bytes(ctypes.byref(args), ctypes.byref(n))
    if st != KDA_OK:
        raise KdaError(st, "kda_bwd_dhu_workspace_bytes")
    return n.value


def kda_bwd_dhu_raw(args: KdaBwdDhuArgs) -> None:
    st = load_library().kda_bwd_dhu(ctypes.byref(args))
    if st != KDA_OK:
        raise KdaError(st, "kda_bwd_dhu")


def kda_bwd_dhu(qg, kg, w, g2, do, dv=None, dht=None, scale=None, cu_seqlens=None, state_dtype=None,
                checkpoint_dtype=None, output_dh0=True, output_checkpoints=True, seg_chunks=0):
    """Reverse state scan of the chunked backward on the current stream.

    Returns (dv2, dhc or None, dh0 or None): dv2 [B, T, HV, V] bf16, dhc [C, HV, K, V]
    (``checkpoint_dtype``: torch.float32 default, or torch.bfloat16) the gradient of
    the state after each chunk (rows as hc of ``kda_fwd``: for varlen ``max_chunks`` rows,
    of which sum_n ceil(len_n/64) are written), dh0 [N, HV, K, V] in
    ``state_dtype`` (torch.float32 default, or torch.bfloat16; dht must match).
    """
    import torch
    if not qg.is_cuda:
        raise RuntimeError("kda_bwd_dhu runs on the GPU only (tensors must be on a HIP device)")
    load_library()
    with torch.cuda.device(qg.device):   # the library launches on the current device
        return _kda_bwd_dhu_on_device(qg, kg, w, g2, do, dv, dht, scale, cu_seqlens, state_dtype, checkpoint_dtype,
                                      output_dh0, output_checkpoints, seg_chunks)


def _kda_bwd_dhu_on_device(qg, kg, w, g2, do, dv, dht, scale, cu_seqlens, state_dtype, checkpoint_dtype,
                           output_dh0, output_checkpoints, seg_chunks):
    import torch
    B, T, HV, K = qg.shape
    V = do.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    sdt = torch.float32 if state_dtype is None else state_dtype
    cdt = torch.float32 if checkpoint_dtype is None else checkpoint_dtype
    for name, dt in (("state_dtype", sdt), ("checkpoint_dtype", cdt)):
        if dt not in (torch.float32, torch.bfloat16):
            raise TypeError(f"{name} must be torch.float32 or torch.bfloat16")
    flags = (KDA_FLAG_STATE_BF16 if sdt == torch.bfloat16 else 0) | (KDA_FLAG_CKPT_BF16 if cdt == torch.bfloat16 else 0)
    dv2 = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=qg.device)
    dh0 = torch.empty((N, HV, K, V), dtype=sdt, device=qg.device) if output_dh0 else None
    dhc = None
    if output_checkpoints:   # varlen: room for the bound, no look at the lengths on the host
        dhc = torch.empty((max_chunks(T, N, B, cu_seqlens is not None), HV, K, V), dtype=cdt, device=qg.device)
    args = make_bwd_args(qg, kg, w, g2, do, dv, dht, scale, cu_seqlens, dv2, dh0, dhc, flags=flags,
                         seg_chunks=seg_chunks)
    n = kda_bwd_dhu_workspace_bytes(args)
    workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=qg.device)
    args.workspace = workspace.data_ptr()
    args.workspace_bytes = workspace.numel()
    kda_bwd_dhu_raw(args)
    return dv2, dhc, dh0
