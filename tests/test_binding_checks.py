"""The Python binding's argument checks (no GPU needed).  The C ABI sees only
pointers and sizes, so the binding is what rejects a tensor whose shape, dtype,
layout or device does not match the others before any kernel could read or write
past it."""
import pytest

torch = pytest.importorskip("torch")

from gated_delta_rule_chunked_amd import kda as K  # noqa: E402

BF = torch.bfloat16


def fwd_tensors(B=1, T=100, HQK=2, HV=4, Kd=64, V=32, N=None, device="cpu"):
    N = B if N is None else N
    z = lambda *s, dt=BF: torch.zeros(s, dtype=dt, device=device)  # noqa: E731
    return dict(q=z(B, T, HQK, Kd), k=z(B, T, HQK, Kd), v=z(B, T, HV, V), g=z(B, T, HV, Kd), beta=z(B, T, HV),
                h0=z(N, HV, Kd, V, dt=torch.float32), o=z(B, T, HV, V), ht=z(N, HV, Kd, V, dt=torch.float32))


def make(**over):
    t = fwd_tensors()
    t.update(over)
    return K.make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], None, t["h0"], t.get("cu_seqlens"), t["o"],
                       t["ht"], hc=t.get("hc"))


def test_well_formed_cpu_tensors_are_refused_for_the_device_only():
    with pytest.raises(ValueError, match="HIP device"):
        make()


@pytest.mark.parametrize("name,shape", [
    ("k", (1, 100, 2, 32)),       # K differs from q
    ("k", (1, 99, 2, 64)),        # T differs
    ("v", (1, 100, 4, 32, 1)),    # wrong rank
    ("g", (1, 100, 2, 64)),       # per q/k head instead of per value head
    ("g", (1, 99, 4, 64)),        # short: the kernels would read past it
    ("beta", (1, 100, 2)),
    ("beta", (1, 100, 4, 1)),
    ("o", (1, 100, 4, 16)),       # short output: the kernels would write past it
    ("h0", (1, 4, 64, 16)),
    ("ht", (2, 4, 64, 32)),
])
def test_shape_mismatch_is_refused(name, shape):
    dt = torch.float32 if name in ("h0", "ht") else BF
    with pytest.raises(ValueError, match=name):
        make(**{name: torch.zeros(shape, dtype=dt)})


def test_dtype_and_layout_are_checked():
    with pytest.raises(TypeError, match="g must be"):
        make(g=torch.zeros((1, 100, 4, 64), dtype=torch.float32))
    with pytest.raises(TypeError, match="ht must be"):
        make(ht=torch.zeros((1, 4, 64, 32), dtype=BF))
    with pytest.raises(ValueError, match="contiguous"):
        make(v=torch.zeros((1, 100, 32, 4), dtype=BF).transpose(2, 3))


def test_tensors_on_another_device_are_refused():
    # cu_seqlens left on another device than q (a host copy is the usual mistake)
    t = fwd_tensors(N=3)
    cu = torch.tensor([0, 30, 60, 100], dtype=torch.int64, device="meta")
    with pytest.raises(ValueError, match="cu_seqlens is on meta"):
        K.make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], None, t["h0"], cu, t["o"], t["ht"])


def test_chunk_states_need_room_for_every_chunk():
    C = (100 + 63) // 64
    with pytest.raises(ValueError, match="hc must have shape"):
        make(hc=torch.zeros((C - 1, 4, 64, 32)))
    # varlen: at least ceil(T/64) + N rows (the chunk total is not known on the host)
    t = fwd_tensors(N=3)
    cu = torch.tensor([0, 30, 60, 100], dtype=torch.int64)
    bound = K.max_chunks(100, 3, 1, varlen=True)
    assert bound == C + 3
    with pytest.raises(ValueError, match="hc must have shape"):
        K.make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], None, t["h0"], cu, t["o"], t["ht"],
                    hc=torch.zeros((bound - 1, 4, 64, 32)))
    with pytest.raises(ValueError, match="HIP device"):
        K.make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], None, t["h0"], cu, t["o"], t["ht"],
                    hc=torch.zeros((bound, 4, 64, 32)))


def test_backward_shapes_are_checked():
    z = lambda *s, dt=BF: torch.zeros(s, dtype=dt)  # noqa: E731
    qg, kg, w, do = z(1, 100, 4, 64), z(1, 100, 4, 64), z(1, 100, 4, 64), z(1, 100, 4, 32)
    g2 = z(1, 100, 4, 64, dt=torch.float32)
    with pytest.raises(ValueError, match="HIP device"):
        K.make_bwd_args(qg, kg, w, g2, do)
    with pytest.raises(ValueError, match="w must have shape"):
        K.make_bwd_args(qg, kg, z(1, 100, 4, 32), g2, do)
    with pytest.raises(ValueError, match="dv2 must have shape"):
        K.make_bwd_args(qg, kg, w, g2, do, dv2=z(1, 99, 4, 32))
    with pytest.raises(TypeError, match="g2 must be"):
        K.make_bwd_args(qg, kg, w, z(1, 100, 4, 64), do)


def test_gpu_entry_points_refuse_host_tensors():
    t = fwd_tensors()
    with pytest.raises(RuntimeError, match="GPU only"):
        K.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"])


def test_missing_library_fails_loudly():
    # a fresh process whose library path does not exist: the binding raises, it never
    # falls back to anything else
    import subprocess
    import sys
    code = ("import gated_delta_rule_chunked_amd.kda as K\n"
            "try:\n"
            "    K.load_library('/nonexistent/libkda.so')\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('loaded')\n")
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "missing" in r.stdout
