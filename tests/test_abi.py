"""The C ABI without a GPU: the library loads, exports every function include/gdn.h declares, and
rejects every bad argument before touching the device (validation precedes any HIP call, so the
fake pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import gated_deltanet_linear_delta_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, UNSUP, ALIGN, WS, ALIAS, NODEV, LAUNCH = range(9)


def header_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_exported():
    lib = gdn.load_library()
    names = header_functions()
    assert set(names) == set(gdn.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n
    # and nothing of the oracle leaked into the product library
    with pytest.raises(AttributeError):
        getattr(lib, "gdn_oracle_recurrent")


def test_debug_library_exports():
    """libgdn_debug.so exports every gdn.h function and the one call of gdn_debug.h; the release
    library does not export the debug call."""
    src = open(os.path.join(ROOT, "include", "gdn_debug.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    debug_names = sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", src)))
    assert debug_names == ["gdn_debug_self_test", "gdn_debug_take_flags"]
    dbg = gdn.load_library("debug")
    for n in header_functions() + debug_names:
        assert hasattr(dbg, n), n
    for n in debug_names:
        with pytest.raises(AttributeError):
            getattr(gdn.load_library(), n)
    assert dbg.gdn_debug_self_test(32) == -1 and dbg.gdn_debug_self_test(-1) == -1   # no device touched


def test_status_strings_and_queries():
    for s in range(9):
        assert gdn.gdn_status_string(s)
    assert gdn.gdn_status_string(1234) == "unknown status"
    # split matrix-core path (few chains): 13,568 bytes per (batch row, value head, chunk) plus
    # 64 * dk * 2 bytes per (batch row, query/key head, chunk)
    per_chunk = 32 * 13568 + 16 * 64 * 128 * 2
    assert gdn.gdn_chunk_fwd_workspace_bytes(1, 4096, 16, 32, 128, 128, 64, gdn.GDN_BF16) == 64 * per_chunk
    assert gdn.gdn_chunk_fwd_workspace_bytes(1, 4097, 16, 32, 128, 128, 64, gdn.GDN_BF16) == 65 * per_chunk
    assert gdn.gdn_chunk_fwd_kernel_name(1, 4096, 16, 32, 128, 128, 64, gdn.GDN_BF16) == "mfma_split"
    # pipelined fused path (many chains) and the float32 path need none
    assert gdn.gdn_chunk_fwd_workspace_bytes(8, 8192, 16, 32, 128, 128, 64, gdn.GDN_BF16) == 0
    assert gdn.gdn_chunk_fwd_kernel_name(8, 8192, 16, 32, 128, 128, 64, gdn.GDN_BF16) == "mfma_pipe"
    assert gdn.gdn_chunk_fwd_workspace_bytes(1, 4096, 16, 32, 128, 128, 64, gdn.GDN_F32) == 0
    assert gdn.gdn_chunk_fwd_workspace_bytes(1, 4096, 16, 33, 128, 128, 64, gdn.GDN_BF16) == 0
    assert gdn.gdn_chunk_fwd_kernel_name(1, 128, 2, 2, 32, 32, 16, gdn.GDN_F32) == "mfma_f32"
    assert gdn.gdn_chunk_fwd_kernel_name(1, 128, 2, 3, 32, 32, 16, gdn.GDN_F32) is None
    assert gdn.gdn_chunk_fwd_kernel_name(1, 128, 2, 2, 48, 32, 16, gdn.GDN_F32) is None


# fake, 16-byte aligned, non-overlapping device addresses (never dereferenced)
BASE = 0x7F0000000000
STRIDE = 1 << 36


def fake(n):
    return ctypes.c_void_p(BASE + n * STRIDE)


def chunk_call(**over):
    lib = gdn.load_library()
    a = dict(q=fake(0), k=fake(1), v=fake(2), g=fake(3), beta=fake(4), s0=fake(5), sf=fake(6), o=fake(7),
             B=2, T=100, Hqk=2, Hv=4, dk=64, dv=32, chunk=32, dtype=gdn.GDN_BF16, scale=1.0,
             ws=None, wsb=0, stream=None)
    a.update(over)
    return lib.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["sf"], a["o"],
                             a["B"], a["T"], a["Hqk"], a["Hv"], a["dk"], a["dv"], a["chunk"], a["dtype"],
                             a["scale"], a["ws"], a["wsb"], a["stream"])


def step_call(**over):
    lib = gdn.load_library()
    a = dict(q=fake(0), k=fake(1), v=fake(2), g=fake(3), beta=fake(4), state=fake(5), o=fake(7),
             B=3, Hqk=2, Hv=4, dk=128, dv=64, dtype=gdn.GDN_F32, scale=1.0, stream=None)
    a.update(over)
    return lib.gdn_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], a["o"], a["B"],
                                  a["Hqk"], a["Hv"], a["dk"], a["dv"], a["dtype"], a["scale"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(g=None), NULL),
    (dict(beta=None), NULL), (dict(o=None), NULL),
    (dict(B=-1), SHAPE), (dict(T=-5), SHAPE), (dict(Hqk=0), SHAPE), (dict(Hv=6, Hqk=4), SHAPE),
    (dict(dk=0), SHAPE), (dict(chunk=0), SHAPE),
    (dict(dk=96), UNSUP), (dict(dv=256), UNSUP), (dict(chunk=128), UNSUP), (dict(chunk=8), UNSUP),
    (dict(dtype=7), UNSUP),
    (dict(q=ctypes.c_void_p(BASE + 8)), ALIGN), (dict(s0=ctypes.c_void_p(BASE + 5 * STRIDE + 4)), ALIGN),
    (dict(beta=ctypes.c_void_p(BASE + 4 * STRIDE + 1)), ALIGN),
    (dict(o=fake(2)), ALIAS), (dict(o=ctypes.c_void_p(BASE + 64)), ALIAS),
    (dict(sf=fake(7)), ALIAS), (dict(sf=fake(0)), ALIAS),
    (dict(sf=ctypes.c_void_p(BASE + 5 * STRIDE + 256)), ALIAS),  # partial overlap with s0
    (dict(o=fake(5)), ALIAS),
])
def test_chunk_fwd_rejects(over, status):
    assert chunk_call(**over) == status


def test_chunk_fwd_empty_batch_is_noop():
    assert chunk_call(B=0, q=None, k=None, v=None, g=None, beta=None, o=None, s0=None, sf=None) == OK


@pytest.mark.parametrize("over,status", [
    (dict(state=None), NULL), (dict(o=None), NULL), (dict(q=None), NULL),
    (dict(B=-2), SHAPE), (dict(Hv=3), SHAPE), (dict(dk=16), UNSUP), (dict(dtype=2), UNSUP),
    (dict(v=ctypes.c_void_p(BASE + 2 * STRIDE + 2)), ALIGN), (dict(g=ctypes.c_void_p(BASE + 3 * STRIDE + 2)), ALIGN),
    (dict(o=fake(5)), ALIAS), (dict(state=fake(1)), ALIAS), (dict(o=fake(3)), ALIAS),
])
def test_recurrent_step_rejects(over, status):
    assert step_call(**over) == status


def test_recurrent_step_empty_batch_is_noop():
    assert step_call(B=0) == OK


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="valid calls on fake pointers are only safe where no device exists")
def test_valid_calls_report_no_device():
    assert chunk_call() == NODEV
    assert chunk_call(sf=fake(5)) == NODEV  # in-place final state is allowed
    assert chunk_call(T=0, o=None) == NODEV
    assert step_call() == NODEV
    assert step_call(g=ctypes.c_void_p(BASE + 3 * STRIDE + 4)) == NODEV  # 4-byte aligned gates are fine


@pytest.mark.skipif(_has_gpu(), reason="needs a host without a GPU")
def test_workspace_check_precedes_device():
    assert chunk_call(wsb=0, ws=None) == NODEV


# the split matrix-core path (bf16, chunk 64, few chains) needs a workspace
SPLIT = dict(dk=128, dv=128, chunk=64, T=100)
SPLIT_WS = 2 * 2 * (4 * 13568 + 2 * 64 * 128 * 2)


def test_split_workspace_size():
    assert gdn.gdn_chunk_fwd_kernel_name(2, 100, 2, 4, 128, 128, 64, gdn.GDN_BF16) == "mfma_split"
    assert gdn.gdn_chunk_fwd_workspace_bytes(2, 100, 2, 4, 128, 128, 64, gdn.GDN_BF16) == SPLIT_WS


@pytest.mark.parametrize("over,status", [
    (dict(ws=fake(8), wsb=SPLIT_WS - 1), WS), (dict(ws=None, wsb=0), WS),
    (dict(ws=None, wsb=SPLIT_WS), NULL),
    (dict(ws=ctypes.c_void_p(BASE + 8 * STRIDE + 8), wsb=SPLIT_WS), ALIGN),
    (dict(ws=fake(0), wsb=SPLIT_WS), ALIAS), (dict(ws=fake(7), wsb=SPLIT_WS), ALIAS),
    (dict(ws=ctypes.c_void_p(BASE + 6 * STRIDE - 4096), wsb=SPLIT_WS), ALIAS),  # runs into sf
])
def test_split_workspace_rejects(over, status):
    assert chunk_call(**SPLIT, **over) == status


@pytest.mark.skipif(_has_gpu(), reason="valid calls on fake pointers are only safe where no device exists")
def test_split_valid_call_reports_no_device():
    assert chunk_call(**SPLIT, ws=fake(8), wsb=SPLIT_WS) == NODEV


# ---------------------------------------------------------------- layer steps around the recurrence


def prologue_call(**over):
    lib = gdn.load_library()
    a = dict(q_in=fake(0), k_in=fake(1), v_in=fake(2), wq=fake(3), wk=fake(4), wv=fake(5), si=fake(6),
             so=fake(7), q=fake(8), k=fake(9), v=fake(10), B=2, T=70, Hqk=2, Hv=4, dk=128, dv=64, W=4,
             dtype=gdn.GDN_BF16, eps=1e-6, stream=None)
    a.update(over)
    return lib.gdn_qkv_prologue(a["q_in"], a["k_in"], a["v_in"], a["wq"], a["wk"], a["wv"], a["si"], a["so"],
                                a["q"], a["k"], a["v"], a["B"], a["T"], a["Hqk"], a["Hv"], a["dk"], a["dv"],
                                a["W"], a["dtype"], a["eps"], a["stream"])


def rmsnorm_call(**over):
    lib = gdn.load_library()
    a = dict(o=fake(0), z=fake(1), w=fake(2), per_head=0, y=fake(3), B=2, T=70, Hv=4, dv=128,
             dtype=gdn.GDN_BF16, eps=1e-6, stream=None)
    a.update(over)
    return lib.gdn_gated_rmsnorm(a["o"], a["z"], a["w"], a["per_head"], a["y"], a["B"], a["T"], a["Hv"],
                                 a["dv"], a["dtype"], a["eps"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q_in=None), NULL), (dict(wv=None), NULL), (dict(k=None), NULL),
    (dict(B=-1), SHAPE), (dict(T=-1), SHAPE), (dict(W=0), SHAPE), (dict(Hv=0), SHAPE),
    (dict(W=5), UNSUP), (dict(dk=48), UNSUP), (dict(dv=256), UNSUP), (dict(dtype=3), UNSUP),
    (dict(eps=-1.0), UNSUP), (dict(eps=float("nan")), UNSUP),
    (dict(q=ctypes.c_void_p(BASE + 8 * STRIDE + 8)), ALIGN), (dict(wk=ctypes.c_void_p(BASE + 4 * STRIDE + 2)), ALIGN),
    (dict(q=fake(0)), ALIAS), (dict(v=fake(5)), ALIAS), (dict(so=fake(6)), ALIAS),
    (dict(k=ctypes.c_void_p(BASE + 8 * STRIDE + 4096)), ALIAS),   # k runs into q
    (dict(so=fake(10)), ALIAS),
])
def test_qkv_prologue_rejects(over, status):
    assert prologue_call(**over) == status


def test_qkv_prologue_noops():
    assert prologue_call(B=0, q_in=None, q=None) == OK
    assert prologue_call(T=0, so=None, q_in=None, q=None) == OK       # nothing to write
    assert prologue_call(T=0, W=1, q_in=None) == OK                   # a width-1 conv has no state


@pytest.mark.parametrize("over,status", [
    (dict(o=None), NULL), (dict(w=None), NULL), (dict(y=None), NULL),
    (dict(B=-1), SHAPE), (dict(per_head=2), SHAPE), (dict(Hv=0), SHAPE),
    (dict(dv=96), UNSUP), (dict(dtype=9), UNSUP), (dict(eps=-0.5), UNSUP),
    (dict(z=ctypes.c_void_p(BASE + STRIDE + 4)), ALIGN), (dict(w=ctypes.c_void_p(BASE + 2 * STRIDE + 1)), ALIGN),
    (dict(y=ctypes.c_void_p(BASE + 256)), ALIAS), (dict(y=fake(2)), ALIAS),
])
def test_gated_rmsnorm_rejects(over, status):
    assert rmsnorm_call(**over) == status


def test_gated_rmsnorm_noops():
    assert rmsnorm_call(T=0, o=None) == OK
    assert rmsnorm_call(B=0, o=None) == OK


@pytest.mark.skipif(_has_gpu(), reason="valid calls on fake pointers are only safe where no device exists")
def test_layer_steps_valid_calls_report_no_device():
    assert prologue_call() == NODEV
    assert prologue_call(si=None, so=None) == NODEV
    assert prologue_call(T=0) == NODEV                                  # writes the state out
    assert rmsnorm_call() == NODEV
    assert rmsnorm_call(y=fake(0)) == NODEV                             # in place over o
    assert rmsnorm_call(y=fake(1), per_head=1) == NODEV                 # in place over z


# ------------------------------------------------------- prefill followed by the gated RMSNorm

GATED_WS = 2 * 100 * 4 * 32 * 2   # float32-vector path: no recurrence workspace, then O in bf16


def gated_call(**over):
    lib = gdn.load_library()
    a = dict(q=fake(0), k=fake(1), v=fake(2), g=fake(3), beta=fake(4), s0=fake(5), sf=fake(6), z=fake(7),
             w=fake(8), per_head=0, eps=1e-6, y=fake(9), B=2, T=100, Hqk=2, Hv=4, dk=64, dv=32, chunk=32,
             dtype=gdn.GDN_BF16, scale=1.0, ws=fake(10), wsb=GATED_WS, stream=None)
    a.update(over)
    return lib.gdn_chunk_fwd_gated(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["sf"], a["z"], a["w"],
                                   a["per_head"], a["eps"], a["y"], a["B"], a["T"], a["Hqk"], a["Hv"], a["dk"],
                                   a["dv"], a["chunk"], a["dtype"], a["scale"], a["ws"], a["wsb"], a["stream"])


def test_gated_workspace_size():
    ws = gdn.gdn_chunk_fwd_gated_workspace_bytes
    # fused matrix-core path with whole value heads per workgroup: the norm runs inside, no O
    assert ws(8, 8192, 16, 32, 128, 128, 64, gdn.GDN_BF16) == 0
    assert ws(8, 100, 16, 32, 128, 64, 64, gdn.GDN_BF16) == 0
    # split path: its own workspace, rounded up to 256 bytes, then O
    per_chunk = 32 * 13568 + 16 * 64 * 128 * 2
    base = 65 * per_chunk
    assert ws(1, 4097, 16, 32, 128, 128, 64, gdn.GDN_BF16) == (base + 255) // 256 * 256 + 4097 * 32 * 128 * 2
    # float32 path: O only
    assert ws(1, 4096, 16, 32, 128, 128, 64, gdn.GDN_F32) == 4096 * 32 * 128 * 4
    assert ws(2, 100, 2, 4, 64, 32, 32, gdn.GDN_BF16) == GATED_WS
    assert ws(1, 0, 16, 32, 128, 128, 64, gdn.GDN_BF16) == 0
    assert ws(1, 4096, 16, 33, 128, 128, 64, gdn.GDN_BF16) == 0      # invalid sizes


@pytest.mark.parametrize("over,status", [
    (dict(z=None), NULL), (dict(w=None), NULL), (dict(y=None), NULL), (dict(q=None), NULL),
    (dict(ws=None), NULL),
    (dict(B=-1), SHAPE), (dict(per_head=2), SHAPE), (dict(Hv=3), SHAPE),
    (dict(dv=96), UNSUP), (dict(chunk=128), UNSUP), (dict(eps=-1.0), UNSUP), (dict(eps=float("nan")), UNSUP),
    (dict(wsb=GATED_WS - 1), WS),
    (dict(z=ctypes.c_void_p(BASE + 7 * STRIDE + 8)), ALIGN), (dict(y=ctypes.c_void_p(BASE + 9 * STRIDE + 4)), ALIGN),
    (dict(w=ctypes.c_void_p(BASE + 8 * STRIDE + 2)), ALIGN),
    (dict(y=fake(2)), ALIAS), (dict(y=fake(8)), ALIAS), (dict(y=fake(5)), ALIAS), (dict(y=fake(6)), ALIAS),
    (dict(y=ctypes.c_void_p(BASE + 7 * STRIDE + 512)), ALIAS),     # partly over z
    (dict(sf=fake(7)), ALIAS), (dict(sf=ctypes.c_void_p(BASE + 5 * STRIDE + 256)), ALIAS),
    (dict(ws=fake(9)), ALIAS), (dict(ws=ctypes.c_void_p(BASE + 8 * STRIDE - 1024)), ALIAS),   # runs into w
])
def test_chunk_fwd_gated_rejects(over, status):
    assert gated_call(**over) == status


def test_chunk_fwd_gated_noops():
    assert gated_call(B=0, q=None, z=None, y=None, ws=None, wsb=0) == OK


@pytest.mark.skipif(_has_gpu(), reason="valid calls on fake pointers are only safe where no device exists")
def test_chunk_fwd_gated_valid_calls_report_no_device():
    assert gated_call() == NODEV
    assert gated_call(y=fake(7)) == NODEV                         # in place over z
    assert gated_call(sf=fake(5)) == NODEV                        # in-place final state
    assert gated_call(T=0, q=None, z=None, y=None, ws=None, wsb=0) == NODEV
    assert gated_call(per_head=1, s0=None, sf=None) == NODEV


# ------------------------------------------------------------------------------ backward

BWD_WS = 2 * 4 * 4 * (2 * 64 * 32 + 4 * 32 * 32 + 2 * 32) * 4     # B * Hv * ceil(100 / 32) * (2 dk dv + 4 * 32 * 32 + 2 * 32) * 4


def bwd_call(**over):
    lib = gdn.load_library()
    a = dict(q=fake(0), k=fake(1), v=fake(2), g=fake(3), beta=fake(4), s0=fake(5), do=fake(6), dsf=fake(7),
             dq=fake(8), dk=fake(9), dv=fake(10), dg=fake(11), dbeta=fake(12), ds0=fake(13), B=2, T=100, Hqk=2,
             Hv=4, dk_=64, dv_=32, dtype=gdn.GDN_BF16, scale=1.0, ws=fake(14), wsb=BWD_WS, stream=None)
    a.update(over)
    return lib.gdn_chunk_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["do"], a["dsf"], a["dq"], a["dk"],
                             a["dv"], a["dg"], a["dbeta"], a["ds0"], a["B"], a["T"], a["Hqk"], a["Hv"], a["dk_"],
                             a["dv_"], a["dtype"], a["scale"], a["ws"], a["wsb"], a["stream"])


def test_bwd_workspace_size():
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 100, 2, 4, 64, 32, gdn.GDN_BF16) == BWD_WS
    assert gdn.gdn_chunk_bwd_workspace_bytes(1, 4096, 16, 32, 128, 128, gdn.GDN_BF16) == 32 * 128 * (2 * 128 * 128 + 4 * 32 * 32 + 2 * 32) * 4
    assert gdn.gdn_chunk_bwd_workspace_bytes(1, 0, 16, 32, 128, 128, gdn.GDN_BF16) == 0
    assert gdn.gdn_chunk_bwd_workspace_bytes(1, 64, 16, 33, 128, 128, gdn.GDN_BF16) == 0


@pytest.mark.parametrize("over,status", [
    (dict(q=None), NULL), (dict(do=None), NULL), (dict(dq=None), NULL), (dict(dg=None), NULL),
    (dict(dbeta=None), NULL), (dict(ws=None), NULL),
    (dict(B=-1), SHAPE), (dict(Hv=3), SHAPE), (dict(T=-2), SHAPE),
    (dict(dk_=48), UNSUP), (dict(dtype=5), UNSUP),
    (dict(wsb=BWD_WS - 1), WS),
    (dict(do=ctypes.c_void_p(BASE + 6 * STRIDE + 8)), ALIGN), (dict(dq=ctypes.c_void_p(BASE + 8 * STRIDE + 4)), ALIGN),
    (dict(dg=ctypes.c_void_p(BASE + 11 * STRIDE + 2)), ALIGN), (dict(ws=ctypes.c_void_p(BASE + 14 * STRIDE + 8)), ALIGN),
    (dict(dq=fake(0)), ALIAS), (dict(dv=fake(6)), ALIAS), (dict(ds0=fake(5)), ALIAS), (dict(ds0=fake(7)), ALIAS),
    (dict(dk=fake(8)), ALIAS), (dict(ws=fake(13)), ALIAS),
    (dict(dbeta=ctypes.c_void_p(BASE + 11 * STRIDE + 64)), ALIAS),        # runs into dg
])
def test_chunk_bwd_rejects(over, status):
    assert bwd_call(**over) == status


def test_chunk_bwd_noops():
    assert bwd_call(B=0, q=None, do=None, dq=None, ws=None, wsb=0) == OK


@pytest.mark.skipif(_has_gpu(), reason="valid calls on fake pointers are only safe where no device exists")
def test_chunk_bwd_valid_calls_report_no_device():
    assert bwd_call() == NODEV
    assert bwd_call(s0=None, dsf=None, ds0=None) == NODEV
    assert bwd_call(T=0, q=None, do=None, dq=None, dg=None, ws=None, wsb=0) == NODEV
    assert bwd_call(dtype=gdn.GDN_F32) == NODEV


# ------------------------------------------------------------------- Kimi Delta Attention

def kda_call(**over):
    lib = gdn.load_library()
    a = dict(q=fake(0), k=fake(1), v=fake(2), g=fake(3), beta=fake(4), s0=fake(5), sf=fake(6), o=fake(7),
             B=2, T=100, Hqk=2, Hv=4, dk_=64, dv_=32, chunk=32, dtype=gdn.GDN_BF16, scale=1.0, ws=None, wsb=0,
             stream=None)
    a.update(over)
    return lib.gdn_kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["sf"], a["o"], a["B"],
                                 a["T"], a["Hqk"], a["Hv"], a["dk_"], a["dv_"], a["chunk"], a["dtype"], a["scale"],
                                 a["ws"], a["wsb"], a["stream"])


KDA_WS = 2 * 4 * 2 * (3 * 64 * 64 * 2 + 2 * 64 * 64 * 2 + 64 * 4 + 64 * 4)   # B Hv ceil(100/64), dk 64


def test_kda_workspace_size():
    assert gdn.gdn_kda_chunk_fwd_workspace_bytes(2, 100, 2, 4, 64, 32, 32, gdn.GDN_BF16) == 0
    assert gdn.gdn_kda_chunk_fwd_workspace_bytes(2, 100, 2, 4, 64, 64, 64, gdn.GDN_BF16) == KDA_WS
    assert gdn.gdn_kda_chunk_fwd_workspace_bytes(2, 100, 2, 4, 64, 64, 64, gdn.GDN_F32) == 0    # unsupported


@pytest.mark.parametrize("over,status", [
    (dict(q=None), NULL), (dict(g=None), NULL), (dict(o=None), NULL),
    (dict(B=-1), SHAPE), (dict(Hv=3), SHAPE), (dict(chunk=0), SHAPE),
    (dict(chunk=128), UNSUP), (dict(chunk=8), UNSUP), (dict(dk_=96), UNSUP), (dict(dtype=4), UNSUP),
    (dict(chunk=64), UNSUP), (dict(chunk=64, dv_=64, dtype=gdn.GDN_F32), UNSUP),
    (dict(chunk=64, dv_=64), WS), (dict(chunk=64, dv_=64, wsb=KDA_WS), NULL),
    (dict(chunk=64, dv_=64, ws=fake(2), wsb=KDA_WS), ALIAS),
    (dict(q=ctypes.c_void_p(BASE + 8)), ALIGN), (dict(g=ctypes.c_void_p(BASE + 3 * STRIDE + 2)), ALIGN),
    (dict(o=fake(3)), ALIAS), (dict(o=ctypes.c_void_p(BASE + 3 * STRIDE + 4096)), ALIAS),   # runs into g
    (dict(sf=fake(7)), ALIAS), (dict(sf=ctypes.c_void_p(BASE + 5 * STRIDE + 256)), ALIAS),
])
def test_kda_rejects(over, status):
    assert kda_call(**over) == status


def test_kda_noops():
    assert kda_call(B=0, q=None, o=None) == OK


@pytest.mark.skipif(_has_gpu(), reason="valid calls on fake pointers are only safe where no device exists")
def test_kda_valid_calls_report_no_device():
    assert kda_call() == NODEV
    assert kda_call(sf=fake(5)) == NODEV
    assert kda_call(T=0, q=None, o=None) == NODEV
    assert kda_call(chunk=16, dtype=gdn.GDN_F32) == NODEV
    assert kda_call(chunk=64, dv_=64, ws=fake(9), wsb=KDA_WS) == NODEV


# ------------------------------------------------------------------------- packed sequences

def varlen_call(**over):
    lib = gdn.load_library()
    a = dict(q=fake(0), k=fake(1), v=fake(2), g=fake(3), beta=fake(4), s0=fake(5), sf=fake(6), o=fake(7),
             cu=fake(8), N=3, maxT=100, total=250, Hqk=2, Hv=4, dk_=64, dv_=32, chunk=32, dtype=gdn.GDN_BF16,
             scale=1.0, ws=None, wsb=0, stream=None)
    a.update(over)
    return lib.gdn_chunk_fwd_varlen(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["sf"], a["o"], a["cu"],
                                    a["N"], a["maxT"], a["total"], a["Hqk"], a["Hv"], a["dk_"], a["dv_"], a["chunk"],
                                    a["dtype"], a["scale"], a["ws"], a["wsb"], a["stream"])


def test_varlen_workspace_size():
    # the split path's workspace for N rows of max_seqlen tokens
    assert gdn.gdn_chunk_fwd_varlen_workspace_bytes(3, 100, 2, 4, 128, 128, 64, gdn.GDN_BF16) == \
        gdn.gdn_chunk_fwd_workspace_bytes(3, 100, 2, 4, 128, 128, 64, gdn.GDN_BF16) > 0
    assert gdn.gdn_chunk_fwd_varlen_workspace_bytes(3, 100, 2, 4, 64, 32, 32, gdn.GDN_BF16) == 0


@pytest.mark.parametrize("over,status", [
    (dict(cu=None), NULL), (dict(q=None), NULL), (dict(o=None), NULL),
    (dict(N=-1), SHAPE), (dict(maxT=-1), SHAPE), (dict(total=-1), SHAPE), (dict(Hv=3), SHAPE),
    (dict(dk_=48), UNSUP), (dict(chunk=128), UNSUP),
    (dict(cu=ctypes.c_void_p(BASE + 8 * STRIDE + 2)), ALIGN), (dict(o=ctypes.c_void_p(BASE + 7 * STRIDE + 4)), ALIGN),
    (dict(o=fake(8)), ALIAS), (dict(sf=fake(8)), ALIAS), (dict(o=fake(0)), ALIAS),
    (dict(dk_=128, dv_=128, chunk=64, ws=None, wsb=0), WS),
])
def test_varlen_rejects(over, status):
    assert varlen_call(**over) == status


def test_varlen_noops():
    assert varlen_call(N=0, cu=None, q=None) == OK


@pytest.mark.skipif(_has_gpu(), reason="valid calls on fake pointers are only safe where no device exists")
def test_varlen_valid_calls_report_no_device():
    assert varlen_call() == NODEV
    assert varlen_call(total=0, q=None, o=None) == NODEV
    assert varlen_call(sf=fake(5)) == NODEV


# ------------------------------------------------------------------------- affine chunk scan

SCAN_B, SCAN_T, SCAN_HQK, SCAN_HV = 1, 1000, 2, 4   # 16 chunks of 64


def scan_call(**over):
    lib = gdn.load_library()
    ws_need = gdn.gdn_chunk_fwd_scan_workspace_bytes(SCAN_B, SCAN_T, SCAN_HQK, SCAN_HV, 128, 128, 64, gdn.GDN_BF16, 4)
    a = dict(q=fake(0), k=fake(1), v=fake(2), g=fake(3), beta=fake(4), s0=fake(5), sf=fake(6), o=fake(7),
             B=SCAN_B, T=SCAN_T, Hqk=SCAN_HQK, Hv=SCAN_HV, dk_=128, dv_=128, chunk=64, dtype=gdn.GDN_BF16, scale=1.0,
             seg=4, ws=fake(9), wsb=ws_need, stream=None)
    a.update(over)
    return lib.gdn_chunk_fwd_scan(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["sf"], a["o"], a["B"],
                                  a["T"], a["Hqk"], a["Hv"], a["dk_"], a["dv_"], a["chunk"], a["dtype"], a["scale"],
                                  a["seg"], a["ws"], a["wsb"], a["stream"])


def transport_call(**over):
    lib = gdn.load_library()
    ws_need = gdn.gdn_chunk_transport_workspace_bytes(SCAN_B, SCAN_T, SCAN_HQK, SCAN_HV, 128, 128, 64, gdn.GDN_BF16)
    a = dict(q=None, k=fake(1), v=fake(2), g=fake(3), beta=fake(4), m=fake(5), n=fake(6), B=SCAN_B, T=SCAN_T,
             Hqk=SCAN_HQK, Hv=SCAN_HV, dk_=128, dv_=128, chunk=64, dtype=gdn.GDN_BF16, ws=fake(9), wsb=ws_need,
             stream=None)
    a.update(over)
    return lib.gdn_chunk_transport(a["q"], a["k"], a["v"], a["g"], a["beta"], a["m"], a["n"], a["B"], a["T"], a["Hqk"],
                                   a["Hv"], a["dk_"], a["dv_"], a["chunk"], a["dtype"], a["ws"], a["wsb"], a["stream"])


def test_scan_segments_and_workspace():
    B, T, Hqk, Hv = 1, 65536, 16, 48          # 1024 chunks
    seg = lambda s, T=T: gdn.gdn_chunk_fwd_scan_segments(B, T, Hqk, Hv, 128, 128, 64, gdn.GDN_BF16, s)
    assert [seg(s) for s in (1, 2, 3, 4, 7, 1024, 5000)] == [1, 2, 3, 4, 7, 1024, 1024]
    assert seg(7, T=200) == 4                  # 4 chunks: one per segment
    assert seg(3, T=640) == 3                  # 10 chunks: 4 + 4 + 2
    assert seg(3, T=0) == 1 and seg(0) == 0
    assert gdn.gdn_chunk_fwd_scan_segments(B, T, Hqk, Hv, 128, 128, 64, gdn.GDN_F32, 4) == 0
    # operands of the split path, then M and N of all segments but the last, then the entry states
    up = lambda x: (x + 255) // 256 * 256
    # the split path's per-chunk operands (gdn_chunk_fwd's workspace holds, on this shape, also
    # the state its pieces hand on, which the scan does not use)
    split_ops = lambda dk: B * (T // 64) * (Hv * 13568 + Hqk * 64 * dk * 2)
    prep = split_ops(128)
    assert gdn.gdn_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, 128, 128, 64, gdn.GDN_BF16) == prep + B * Hv * 128 * 128 * 4
    chains = B * Hv
    want = up(prep) + 2 * up(chains * 3 * 128 * 128 * 4) + up(chains * 4 * 128 * 128 * 4)
    assert gdn.gdn_chunk_fwd_scan_workspace_bytes(B, T, Hqk, Hv, 128, 128, 64, gdn.GDN_BF16, 4) == want
    assert gdn.gdn_chunk_fwd_scan_workspace_bytes(B, T, Hqk, Hv, 128, 128, 64, gdn.GDN_BF16, 1) == up(prep) + \
        up(chains * 128 * 128 * 4)
    assert gdn.gdn_chunk_fwd_scan_workspace_bytes(B, 0, Hqk, Hv, 128, 128, 64, gdn.GDN_BF16, 4) == 0
    assert gdn.gdn_chunk_fwd_scan_workspace_bytes(B, T, Hqk, Hv, 128, 128, 32, gdn.GDN_BF16, 4) == 0
    assert gdn.gdn_chunk_transport_workspace_bytes(B, T, Hqk, Hv, 64, 128, 64, gdn.GDN_BF16) == up(split_ops(64))


@pytest.mark.parametrize("over,status", [
    (dict(q=None), NULL), (dict(o=None), NULL), (dict(ws=None), NULL),
    (dict(B=-1), SHAPE), (dict(T=-1), SHAPE), (dict(Hv=3), SHAPE), (dict(seg=0), SHAPE),
    (dict(dtype=gdn.GDN_F32), UNSUP), (dict(chunk=32), UNSUP), (dict(dk_=32), UNSUP), (dict(dk_=48), UNSUP),
    (dict(wsb=1024), WS),
    (dict(o=ctypes.c_void_p(BASE + 7 * STRIDE + 4)), ALIGN), (dict(g=ctypes.c_void_p(BASE + 3 * STRIDE + 2)), ALIGN),
    (dict(o=fake(0)), ALIAS), (dict(sf=fake(1)), ALIAS), (dict(ws=fake(2)), ALIAS), (dict(o=fake(6)), ALIAS),
])
def test_scan_rejects(over, status):
    assert scan_call(**over) == status


@pytest.mark.parametrize("over,status", [
    (dict(m=None), NULL), (dict(n=None), NULL), (dict(k=None), NULL), (dict(ws=None), NULL),
    (dict(T=-1), SHAPE), (dict(Hv=3), SHAPE),
    (dict(dtype=gdn.GDN_F32), UNSUP), (dict(chunk=16), UNSUP),
    (dict(wsb=16), WS), (dict(m=ctypes.c_void_p(BASE + 5 * STRIDE + 8)), ALIGN),
    (dict(m=fake(6)), ALIAS), (dict(n=fake(2)), ALIAS), (dict(m=fake(9)), ALIAS),
])
def test_transport_rejects(over, status):
    assert transport_call(**over) == status


def test_scan_transport_noops():
    assert scan_call(B=0, q=None, ws=None, wsb=0) == OK
    assert transport_call(B=0, k=None, ws=None, wsb=0) == OK


@pytest.mark.skipif(_has_gpu(), reason="valid calls on fake pointers are only safe where no device exists")
def test_scan_transport_valid_calls_report_no_device():
    assert scan_call() == NODEV
    assert scan_call(sf=fake(5)) == NODEV                       # in place
    assert scan_call(T=0, ws=None, wsb=0, q=None, o=None) == NODEV
    assert transport_call() == NODEV
    assert transport_call(q=fake(0)) == NODEV
    assert transport_call(T=0, ws=None, wsb=0) == NODEV


def test_chunk_fwd_routes_scarce_long_chains_to_the_scan(monkeypatch, hooks):
    """gdn_chunk_fwd cuts chains into segments by itself when 32-column tiles over dv + dk give at
    most 128 workgroups and every segment keeps at least 8 chunks."""
    name = lambda B, T, Hqk, Hv: gdn.gdn_chunk_fwd_kernel_name(B, T, Hqk, Hv, 128, 128, 64, gdn.GDN_BF16)
    ws = lambda B, T, Hqk, Hv: gdn.gdn_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, 128, 128, 64, gdn.GDN_BF16)
    scan_ws = lambda B, T, Hqk, Hv, p: gdn.gdn_chunk_fwd_scan_workspace_bytes(B, T, Hqk, Hv, 128, 128, 64,
                                                                            gdn.GDN_BF16, p)
    assert name(1, 65536, 2, 6) == "mfma_scan"          # 6 chains: 48 tiles -> 6 segments
    assert ws(1, 65536, 2, 6) == scan_ws(1, 65536, 2, 6, 6)
    assert name(1, 65536, 16, 16) == "mfma_scan"        # 128 tiles -> 3 segments
    assert ws(1, 65536, 16, 16) == scan_ws(1, 65536, 16, 16, 3)
    assert name(1, 65536, 16, 48) == "mfma_split"       # 384 tiles: the chains fill the chip
    assert name(1, 4096, 16, 32) == "mfma_split"        # 256 tiles: 2 segments would not pay
    assert name(1, 2000, 1, 1) == "mfma_split"          # 33 segments would hold under 8 chunks
    assert name(1, 20000, 1, 1) == "mfma_scan"
    monkeypatch.setenv("GDN_SCAN_SEGMENTS", "0")
    assert name(1, 65536, 2, 6) == "mfma_split"
    # the split path's operands and the state its pieces hand on: as large as the one-segment
    # scan's operands and entry states
    assert ws(1, 65536, 2, 6) == gdn.gdn_chunk_fwd_scan_workspace_bytes(1, 65536, 2, 6, 128, 128, 64,
                                                                        gdn.GDN_BF16, 1)


def test_release_library_reads_no_environment(monkeypatch):
    """The route and the workspace size of the release library follow from the arguments alone:
    the overrides that the test-hooks build honours change nothing in libgdn.so."""
    args = (1, 65536, 2, 6, 128, 128, 64, gdn.GDN_BF16)
    name, ws = gdn.gdn_chunk_fwd_kernel_name(*args), gdn.gdn_chunk_fwd_workspace_bytes(*args)
    small = (2, 300, 2, 4, 128, 128, 64, gdn.GDN_BF16)
    name_s = gdn.gdn_chunk_fwd_kernel_name(*small)
    for var, val in (("GDN_SCAN_SEGMENTS", "0"), ("GDN_MFMA_PATH", "fused"), ("GDN_DISABLE_MFMA", "1"),
                     ("GDN_SPLIT_BV", "16"), ("GDN_MFMA_BV", "64")):
        monkeypatch.setenv(var, val)
        assert gdn.gdn_chunk_fwd_kernel_name(*args) == name == "mfma_scan"
        assert gdn.gdn_chunk_fwd_workspace_bytes(*args) == ws
        assert gdn.gdn_chunk_fwd_kernel_name(*small) == name_s == "mfma_split"
    # the test-hooks build does take them
    with gdn.test_hooks():
        assert gdn.gdn_chunk_fwd_kernel_name(*small) == "mfma_f32"
