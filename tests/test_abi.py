"""The C ABI library loads, exports every declared symbol and validates its
arguments on the host (CPU only: no kernel is launched here)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_09_amd._lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libkda.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_signatures():
    assert declared_functions() == sorted(L.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = L.load()
    assert lib.kda_abi_version() == L.ABI_VERSION == 4
    for s in range(8):
        assert lib.kda_status_string(s)
    assert lib.kda_status_string(99) == b"unknown status"


# Fake, aligned, never-dereferenced addresses: validation fails before any HIP call.
P = ctypes.c_void_p(0x10000)
MIS = ctypes.c_void_p(0x10004)


def _device_count():
    try:
        import torch
        return torch.cuda.device_count()    # counts devices without initialising one
    except Exception:
        return 0


# Calls that pass validation go on to launch kernels on the fake addresses above,
# so they only run where no device is visible (the CPU suite).
needs_no_device = pytest.mark.skipif(_device_count() > 0,
                                     reason="passes validation and would launch on fake addresses")


def prefill(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, b=P, init=None, cu=None, N=1, T=64, H=2, dk=64, dv=64, dt=L.KDA_BF16,
             o=P, fin=P)
    a.update(kw)
    return lib.kda_chunk_prefill(a["q"], a["k"], a["v"], a["la"], a["b"], a["init"], a["cu"], a["N"], a["T"],
                                 a["H"], a["dk"], a["dv"], a["dt"], a["o"], a["fin"], None)


def decode(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, b=P, S=P, N=4, H=2, dk=64, dv=64, dt=L.KDA_BF16, o=P)
    a.update(kw)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["la"], a["b"], a["S"], a["N"], a["H"], a["dk"],
                               a["dv"], a["dt"], a["o"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), 3), (dict(dk=96), 2), (dict(dv=32), 2), (dict(H=0), 2), (dict(N=0), 2),
    (dict(T=-1), 2), (dict(N=2), 2), (dict(N=70000, cu=P), 2),
    (dict(q=None), 1), (dict(b=None), 1), (dict(o=None), 1), (dict(la=MIS), 4), (dict(fin=MIS), 4),
    (dict(init=MIS), 4), (dict(cu=MIS, N=1), 4),
])
def test_prefill_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert prefill(L.load(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dt=-1), 3), (dict(dk=32), 2), (dict(H=0), 2), (dict(N=-1), 2),
    (dict(S=None), 1), (dict(v=None), 1), (dict(q=MIS), 4), (dict(S=MIS), 4),
])
def test_decode_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert decode(L.load(), **kw) == code


def prefill_gated(lib, **kw):
    a = dict(q=P, k=P, v=P, z=P, A=P, b=P, init=None, cu=None, N=1, T=64, H=2, dk=64, dv=64, dt=L.KDA_BF16,
             o=P, fin=P)
    a.update(kw)
    return lib.kda_chunk_prefill_gated(a["q"], a["k"], a["v"], a["z"], a["A"], a["b"], a["init"], a["cu"], a["N"],
                                       a["T"], a["H"], a["dk"], a["dv"], a["dt"], a["o"], a["fin"], None)


def decode_gated(lib, **kw):
    a = dict(q=P, k=P, v=P, z=P, A=P, b=P, S=P, N=4, H=2, dk=64, dv=64, dt=L.KDA_BF16, o=P)
    a.update(kw)
    return lib.kda_decode_step_gated(a["q"], a["k"], a["v"], a["z"], a["A"], a["b"], a["S"], a["N"], a["H"],
                                     a["dk"], a["dv"], a["dt"], a["o"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), 3), (dict(dk=96), 2), (dict(N=2), 2),
    (dict(z=None), 1), (dict(A=None), 1), (dict(b=None), 1), (dict(A=MIS), 4), (dict(z=MIS), 4),
])
def test_gated_prefill_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert prefill_gated(L.load(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dt=-1), 3), (dict(dk=32), 2), (dict(A=None), 1), (dict(z=None), 1), (dict(A=MIS), 4),
])
def test_gated_decode_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert decode_gated(L.load(), **kw) == code


def epilogue(lib, **kw):
    a = dict(o=P, g=P, w=None, rows=96, dv=128, eps=1e-5, dt=L.KDA_BF16, y=P)
    a.update(kw)
    return lib.kda_output_gate_rmsnorm(a["o"], a["g"], a["w"], a["rows"], a["dv"], a["eps"], a["dt"], a["y"], None)


def prefill_epi(lib, **kw):
    a = dict(q=P, k=P, v=P, z=P, A=P, b=P, og=P, w=None, eps=1e-5, init=None, cu=None, N=1, T=64, H=2, dk=64,
             dv=64, dt=L.KDA_BF16, y=P, fin=P)
    a.update(kw)
    return lib.kda_chunk_prefill_gated_epilogue(a["q"], a["k"], a["v"], a["z"], a["A"], a["b"], a["og"], a["w"],
                                                a["eps"], a["init"], a["cu"], a["N"], a["T"], a["H"], a["dk"],
                                                a["dv"], a["dt"], a["y"], a["fin"], None)


def decode_epi(lib, **kw):
    a = dict(q=P, k=P, v=P, z=P, A=P, b=P, og=P, w=None, eps=1e-5, S=P, N=4, H=2, dk=64, dv=64, dt=L.KDA_BF16,
             y=P)
    a.update(kw)
    return lib.kda_decode_step_gated_epilogue(a["q"], a["k"], a["v"], a["z"], a["A"], a["b"], a["og"], a["w"],
                                              a["eps"], a["S"], a["N"], a["H"], a["dk"], a["dv"], a["dt"], a["y"],
                                              None)


NAN, INF = float("nan"), float("inf")


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), 3), (dict(dv=96), 2), (dict(rows=-1), 2), (dict(rows=1 << 62), 2), (dict(eps=-1e-5), 7),
    (dict(eps=NAN), 7), (dict(eps=INF), 7), (dict(o=None), 1), (dict(g=None), 1), (dict(y=None), 1),
    (dict(o=MIS), 4), (dict(g=MIS), 4), (dict(y=MIS), 4), (dict(w=MIS), 4),
])
def test_epilogue_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert epilogue(L.load(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), 3), (dict(dv=96), 2), (dict(N=2), 2), (dict(H=0), 2), (dict(T=-1), 2), (dict(eps=-1.0), 7),
    (dict(og=None), 1), (dict(z=None), 1), (dict(A=None), 1), (dict(og=MIS), 4), (dict(w=MIS), 4),
    (dict(y=MIS), 4),
])
def test_prefill_epilogue_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert prefill_epi(L.load(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dt=-1), 3), (dict(dk=32), 2), (dict(eps=NAN), 7), (dict(og=None), 1), (dict(A=None), 1),
    (dict(og=MIS), 4), (dict(w=MIS), 4),
])
def test_decode_epilogue_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert decode_epi(L.load(), **kw) == code


def prologue(lib, **kw):
    a = dict(xq=P, xk=P, xv=P, w=P, si=None, cu=None, N=1, T=64, H=2, dk=64, dv=64, dt=L.KDA_BF16, q=P, k=P, v=P,
             so=None)
    a.update(kw)
    return lib.kda_short_conv_prologue(a["xq"], a["xk"], a["xv"], a["w"], a["si"], a["cu"], a["N"], a["T"], a["H"],
                                       a["dk"], a["dv"], a["dt"], a["q"], a["k"], a["v"], a["so"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), 3), (dict(dk=32), 2), (dict(dv=256), 2), (dict(N=0), 2), (dict(N=2), 2), (dict(H=0), 2),
    (dict(T=-5), 2), (dict(H=70000), 2), (dict(T=1 << 40, H=4096), 2), (dict(xq=None), 1), (dict(w=None), 1),
    (dict(v=None), 1), (dict(xv=MIS), 4), (dict(w=MIS), 4), (dict(si=MIS), 4), (dict(so=MIS), 4),
    (dict(si=P, so=P), 7), (dict(si=ctypes.c_void_p(0x10000), so=ctypes.c_void_p(0x10000 + 16)), 7),
])
def test_prologue_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert prologue(L.load(), **kw) == code


def test_prologue_accepts_adjacent_states():
    # [N, 3, H, C] bf16 with N=1, H=2, C=192: 2304 bytes; a state right after the other is fine
    lib = L.load()
    st = prologue(lib, si=ctypes.c_void_p(0x10000), so=ctypes.c_void_p(0x10000 + 2304))
    assert st in (0, 5)     # no overlap: validation passes (5 = no device here)


def decode_fused(lib, **kw):
    a = dict(xq=P, xk=P, xv=P, w=P, cs=P, z=P, A=P, b=P, og=P, g=None, eps=1e-5, S=P, N=4, H=2, dk=64, dv=64,
             dt=L.KDA_BF16, y=P)
    a.update(kw)
    return lib.kda_decode_step_fused(a["xq"], a["xk"], a["xv"], a["w"], a["cs"], a["z"], a["A"], a["b"], a["og"],
                                     a["g"], a["eps"], a["S"], a["N"], a["H"], a["dk"], a["dv"], a["dt"], a["y"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=9), 3), (dict(dv=48), 2), (dict(H=0), 2), (dict(eps=-0.5), 7), (dict(w=None), 1), (dict(cs=None), 1),
    (dict(og=None), 1), (dict(A=None), 1), (dict(w=MIS), 4), (dict(cs=MIS), 4), (dict(g=MIS), 4),
])
def test_fused_decode_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert decode_fused(L.load(), **kw) == code


def test_empty_calls_are_no_ops():
    lib = L.load()
    assert decode(lib, N=0, q=None, S=None) == 0
    assert prefill(lib, T=0, q=None, k=None, v=None, la=None, b=None, o=None, fin=None) == 0
    assert epilogue(lib, rows=0, o=None, g=None, y=None) == 0
    assert decode_epi(lib, N=0, q=None, S=None, og=None, y=None) == 0
    assert prefill_epi(lib, T=0, q=None, k=None, v=None, z=None, b=None, og=None, y=None, fin=None) == 0
    assert prologue(lib, T=0, xq=None, xk=None, xv=None, w=None, q=None, k=None, v=None) == 0
    assert decode_fused(lib, N=0, xq=None, w=None, cs=None, S=None, y=None) == 0
    assert prefill_split(lib, T=0, q=None, k=None, v=None, la=None, b=None, o=None, fin=None, ws=None) == 0


def _has_gpu():
    import torch
    try:
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device path")
def test_valid_call_without_a_device_reports_no_device():
    assert prefill(L.load()) == 5
    assert decode(L.load()) == 5
    assert prefill_gated(L.load()) == 5
    assert decode_gated(L.load()) == 5
    assert epilogue(L.load()) == 5
    assert prefill_epi(L.load()) == 5
    assert decode_epi(L.load()) == 5
    assert prologue(L.load()) == 5
    assert decode_fused(L.load()) == 5
    assert prefill_split(L.load()) == 5
    assert prefill_split(L.load(), seg=1) == 5


def test_binding_raises_when_library_missing(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        L.load(str(tmp_path / "nope.so"))


def prefill_split(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, b=P, init=None, T=4096, H=2, dk=64, dv=64, dt=L.KDA_BF16, seg=4, ws=P,
             wsb=1 << 40, o=P, fin=P)
    a.update(kw)
    return lib.kda_chunk_prefill_split(a["q"], a["k"], a["v"], a["la"], a["b"], a["init"], a["T"], a["H"], a["dk"],
                                       a["dv"], a["dt"], a["seg"], a["ws"], a["wsb"], a["o"], a["fin"], None)


def prefill_gated_split(lib, **kw):
    a = dict(q=P, k=P, v=P, z=P, A=P, b=P, init=None, T=4096, H=2, dk=64, dv=64, dt=L.KDA_BF16, seg=4, ws=P,
             wsb=1 << 40, o=P, fin=P)
    a.update(kw)
    return lib.kda_chunk_prefill_gated_split(a["q"], a["k"], a["v"], a["z"], a["A"], a["b"], a["init"], a["T"],
                                             a["H"], a["dk"], a["dv"], a["dt"], a["seg"], a["ws"], a["wsb"], a["o"],
                                             a["fin"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), 3), (dict(seg=0), 7), (dict(seg=-3), 7), (dict(dk=96), 2), (dict(H=0), 2), (dict(T=-1), 2),
    (dict(H=70000), 2), (dict(ws=None), 1), (dict(q=None), 1), (dict(o=None), 1),
    (dict(ws=MIS), 4), (dict(la=MIS), 4), (dict(init=MIS), 4), (dict(wsb=1000), 7),
    (dict(H=40000, dk=128, dv=128), 2), (dict(H=20000, dk=64, dv=128, dt=L.KDA_F32), 2),
    # one segment is the plain prefill: its own checks apply and no workspace is needed
    (dict(seg=1, ws=None, q=None), 1), (dict(T=64, seg=8, ws=None, b=None), 1),
])
def test_split_prefill_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert prefill_split(L.load(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), 3), (dict(seg=0), 7), (dict(A=None), 1), (dict(z=None), 1), (dict(A=MIS), 4), (dict(ws=None), 1),
])
def test_gated_split_prefill_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert prefill_gated_split(L.load(), **kw) == code


def test_split_workspace_sizes():
    """End states, transitions and Phi_t^T q_t rows, each padded to 256 bytes; zero for one segment."""
    lib = L.load()
    pad = lambda x: (x + 255) // 256 * 256
    T, H = 4096, 3          # 64 chunks; 4 segments of 16 chunks (1024 tokens)
    for dk, dv, dt, es in [(128, 128, L.KDA_BF16, 2), (128, 64, L.KDA_BF16, 2), (64, 128, L.KDA_F32, 4)]:
        want = pad(4 * H * dk * dv * 4) + pad(3 * H * dk * dk * 4) + pad((T - 1024) * H * dk * es)
        assert lib.kda_split_workspace_bytes(T, H, dk, dv, dt, 4) == want
    # 5 requested segments of 64 chunks: 13 chunks each, which gives 5 segments
    assert lib.kda_split_workspace_bytes(T, 1, 64, 64, L.KDA_BF16, 5) == \
        pad(5 * 64 * 64 * 4) + pad(4 * 64 * 64 * 4) + pad((T - 13 * 64) * 64 * 2)
    # 40 requested segments of 3 chunks: one chunk each, which gives 3
    assert lib.kda_split_workspace_bytes(192, 1, 64, 64, L.KDA_BF16, 40) == \
        pad(3 * 64 * 64 * 4) + pad(2 * 64 * 64 * 4) + pad(128 * 64 * 2)
    for T, seg in [(4096, 1), (64, 4), (0, 4)]:
        assert lib.kda_split_workspace_bytes(T, H, 128, 128, L.KDA_BF16, seg) == 0
    assert lib.kda_split_workspace_bytes(4096, 0, 128, 128, L.KDA_BF16, 4) == 0
    assert lib.kda_split_workspace_bytes(4096, H, 96, 128, L.KDA_BF16, 4) == 0


def test_split_segment_model():
    """The cost model keeps one segment when the heads fill the GPU and splits when few heads
    leave most compute units idle; the count never exceeds the chunk count."""
    lib = L.load()
    assert lib.kda_split_segments(65536, 96, 128, 128, 256) == 1
    assert lib.kda_split_segments(1048576, 96, 128, 128, 256) == 1
    n12 = lib.kda_split_segments(65536, 12, 128, 128, 256)
    n1 = lib.kda_split_segments(65536, 1, 128, 128, 256)
    assert 2 <= n12 < n1
    assert lib.kda_split_segments(200, 1, 64, 64, 256) <= 4
    for bad in [(0, 4, 128, 128, 256), (4096, 0, 128, 128, 256), (4096, 4, 96, 128, 256), (4096, 4, 128, 128, 0)]:
        assert lib.kda_split_segments(*bad) == 1
    # more compute units never ask for fewer segments
    counts = [lib.kda_split_segments(65536, 12, 128, 128, c) for c in (64, 128, 256, 512)]
    assert counts == sorted(counts)


@needs_no_device
def test_split_binding_checks_before_calling_the_library():
    """The split wrapper rejects a wrong initial-state shape or a wrong decay dtype itself, and
    sizes the workspace with the library's own function."""
    import torch
    T, H, d = 256, 2, 64
    q = torch.zeros(T, H, d, dtype=torch.bfloat16)
    la = torch.zeros(T, H, d)
    b = torch.zeros(T, H)
    with pytest.raises(ValueError, match="init_state"):
        L.kda_chunk_prefill_split(q, q, q, la, b, init_state=torch.zeros(2, H, d, d), segments=2)
    with pytest.raises(TypeError, match="decay"):
        L.kda_chunk_prefill_split(q, q, q, la.double(), b, segments=2)
    lib = L.load()
    assert L.split_workspace_bytes(T, H, d, d, torch.bfloat16, 2) == \
        lib.kda_split_workspace_bytes(T, H, d, d, L.KDA_BF16, 2) > 0
    assert L.split_workspace_bytes(T, H, d, d, torch.float32, 1) == 0


# ---- sizes at the edge of one dispatch (blocks x threads < 2^32, blocks < 2^31) ----

OK_OR_NO_DEVICE = (0, 5)    # validation passed: 0 with a device, 5 without one



@needs_no_device
def test_fp32_dk128_is_accepted():
    lib = L.load()
    for dv in (64, 128):
        assert prefill(lib, dt=L.KDA_F32, dk=128, dv=dv) in OK_OR_NO_DEVICE
        assert prefill_gated(lib, dt=L.KDA_F32, dk=128, dv=dv) in OK_OR_NO_DEVICE
        assert prefill_split(lib, dt=L.KDA_F32, dk=128, dv=dv) in OK_OR_NO_DEVICE


@needs_no_device
def test_decode_grid_limit():
    """1024 threads per (sequence, head) pair: at most 4,194,303 pairs; 512 with the prologue."""
    lib = L.load()
    assert decode(lib, N=65535, H=64) in OK_OR_NO_DEVICE           # 4,194,240 pairs
    assert decode(lib, N=65536, H=64) == 2                         # 4,194,304 pairs
    assert decode_fused(lib, N=65536, H=64) in OK_OR_NO_DEVICE     # 512 threads per pair
    assert decode_fused(lib, N=65536, H=128) == 2                  # 8,388,608 pairs


@needs_no_device
def test_prefill_grid_limit():
    """512 threads per workgroup; one workgroup per (sequence, head) pair at d_v = 64,
    two per pair (padded to groups of 16) at d_v = 128."""
    lib = L.load()
    assert prefill(lib, N=65535, H=128, cu=P, dv=64) in OK_OR_NO_DEVICE     # 8,388,480 workgroups
    assert prefill(lib, N=65535, H=129, cu=P, dv=64) == 2                   # 8,454,015
    assert prefill(lib, N=65535, H=64, cu=P, dv=128) in OK_OR_NO_DEVICE     # 8,388,480
    assert prefill(lib, N=65535, H=65, cu=P, dv=128) == 2


@needs_no_device
def test_split_grid_limits():
    """The segment runs and transitions share one launch when d_v = d_k; the
    correction's grid is two workgroups per CU, and it addresses 512 tokens of a
    head with 32-bit byte offsets: 512 H max(d_k, d_v) element bytes < 2^32."""
    lib = L.load()
    # 2 segments x 65535 heads: runs + transitions = 3 x 65535 units x 2 workgroups each
    assert prefill_split(lib, H=65535, dk=128, dv=128, T=4096, seg=2) == 2
    assert prefill_split(lib, H=30000, dk=64, dv=64, T=4096, seg=2) in OK_OR_NO_DEVICE
    # the correction has no grid limit of its own (any length, any segment count)
    assert prefill_split(lib, H=65535, dk=64, dv=64, T=2 * 65600, seg=2) in OK_OR_NO_DEVICE
    # offsets: 512 x 16384 heads x 128 x 4 bytes = 2^32 (fp32, d = 128) is one too many
    assert prefill_split(lib, H=16383, dk=128, dv=128, T=4096, seg=2, dt=L.KDA_F32) in OK_OR_NO_DEVICE
    assert prefill_split(lib, H=16384, dk=128, dv=128, T=4096, seg=2, dt=L.KDA_F32) == 2


@needs_no_device
def test_epilogue_grid_limit():
    """One 64-thread workgroup per 4 rows (bf16, d_v = 128) or 2 rows (fp32, d_v = 128)."""
    lib = L.load()
    per_block = {(L.KDA_BF16, 128): 4, (L.KDA_F32, 128): 2, (L.KDA_BF16, 64): 8, (L.KDA_F32, 64): 4}
    for (dt, dv), rpb in per_block.items():
        limit = rpb * ((2 ** 32 - 1) // 64)
        assert epilogue(lib, dt=dt, dv=dv, rows=limit) in OK_OR_NO_DEVICE
        assert epilogue(lib, dt=dt, dv=dv, rows=limit + 1) == 2


@needs_no_device
def test_prologue_grid_limit():
    """One 64-thread workgroup per 16 tokens of a group of heads (4 heads per group at
    bf16 and d = 128, 2 at fp32 and d = 128)."""
    lib = L.load()
    strips = (2 ** 32 - 1) // 64
    assert prologue(lib, dk=128, dv=128, H=4, T=16 * strips) in OK_OR_NO_DEVICE
    assert prologue(lib, dk=128, dv=128, H=5, T=16 * strips) == 2
    assert prologue(lib, dk=128, dv=128, H=4, T=16 * strips, dt=L.KDA_F32) == 2
    assert prologue(lib, dk=128, dv=128, H=2, T=16 * strips, dt=L.KDA_F32) in OK_OR_NO_DEVICE


def test_wait_giveups_host_path():
    """The give-up counter's query: a NULL output is rejected before any HIP call;
    without a device it reports no device."""
    lib = L.load()
    assert lib.kda_wait_giveups(None, 0, None) == 1
    n = ctypes.c_uint32(7)
    st = lib.kda_wait_giveups(ctypes.byref(n), 1, None)
    if _has_gpu():
        assert st == 0
    else:
        assert st == 5 and n.value == 7


def prefill_split_noalloc(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, b=P, init=None, T=4096, H=2, dk=64, dv=64, dt=L.KDA_BF16, seg=4, o=P, fin=P)
    a.update(kw)
    return lib.kda_chunk_prefill_split_noalloc(a["q"], a["k"], a["v"], a["la"], a["b"], a["init"], a["T"], a["H"],
                                               a["dk"], a["dv"], a["dt"], a["seg"], a["o"], a["fin"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), 3), (dict(seg=0), 7), (dict(dk=96), 2), (dict(H=0), 2), (dict(T=-1), 2), (dict(q=None), 1),
    (dict(o=None), 1), (dict(la=MIS), 4), (dict(init=MIS), 4),
    # a plan beyond the library's scratch: 65,536 tokens x 12 heads x d 128 in 8 segments needs ~200 MB
    (dict(T=65536, H=12, dk=128, dv=128, seg=8), 7),
])
def test_noalloc_split_rejects_bad_arguments_before_touching_the_device(kw, code):
    assert prefill_split_noalloc(L.load(), **kw) == code


@needs_no_device
def test_noalloc_split_scratch_limit():
    """The largest plan the scratch holds passes validation; one byte more does not."""
    lib = L.load()
    assert L.SPLIT_SCRATCH_BYTES == 64 << 20
    # 16,384 tokens in 4 segments, 12 heads, d = 128, bf16: end states 3 MB, transitions 2.4 MB and
    # Phi^T q rows of 12,288 tokens 37.7 MB, under 64 MiB
    need = lib.kda_split_workspace_bytes(16384, 12, 128, 128, L.KDA_BF16, 4)
    assert 0 < need <= L.SPLIT_SCRATCH_BYTES
    assert prefill_split_noalloc(lib, T=16384, H=12, dk=128, dv=128, seg=4) in OK_OR_NO_DEVICE
    # twice the heads is beyond it
    assert lib.kda_split_workspace_bytes(16384, 24, 128, 128, L.KDA_BF16, 4) > L.SPLIT_SCRATCH_BYTES
    assert prefill_split_noalloc(lib, T=16384, H=24, dk=128, dv=128, seg=4) == 7
    assert b"scratch" in lib.kda_last_error()
