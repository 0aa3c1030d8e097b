"""Gated delta rule (Gated DeltaNet core) on AMD MI355X: Python binding of libgdn.so.

The binding only marshals arguments: every step of the computation runs in the HIP kernels of
``libgdn.so`` (built in-tree by ``gated_deltanet_linear_delta_amd/build.py``).  torch tensors
provide device memory and the HIP stream; nothing is computed with torch.  If the library is
missing, every call raises -- there is no fallback path.

Entry points (same names as the C ABI in include/gdn.h):

* :func:`gdn_chunk_fwd` -- prefill, chunkwise, optional initial / final state.
* :func:`gdn_recurrent_step` -- decode, one token per sequence, state updated in place.
* :func:`gdn_qkv_prologue` -- short causal conv, SiLU and q/k L2 norm after the projections.
* :func:`gdn_gated_rmsnorm` -- RMSNorm of the output times SiLU of the gate.
* :func:`gdn_chunk_fwd_gated` -- prefill followed by the gated RMSNorm (fused where it can be).
* :func:`gdn_chunk_bwd` -- backward pass of the prefill (gradients of q, k, v, g, beta, S0).
* :func:`gdn_kda_chunk_fwd` -- Kimi Delta Attention prefill (one decay per key channel).
* :func:`gdn_chunk_fwd_varlen` -- prefill of packed sequences of different lengths.
* :func:`gdn_chunk_fwd_scan` -- prefill with every chain cut into segments (affine chunk scan).
* :func:`gdn_chunk_transport` -- the affine state map (M, N) of a stretch of tokens.
* :func:`gdn_chunk_fwd_workspace_bytes`, :func:`gdn_chunk_fwd_gated_workspace_bytes`,
  :func:`gdn_chunk_fwd_kernel_name`, :func:`gdn_status_string`.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

__all__ = [
    "GDN_F32", "GDN_BF16", "GdnError", "library_path", "load_library", "gdn_chunk_fwd",
    "gdn_recurrent_step", "gdn_chunk_fwd_workspace_bytes", "gdn_chunk_fwd_kernel_name",
    "gdn_status_string", "gdn_qkv_prologue", "gdn_gated_rmsnorm", "gdn_chunk_fwd_gated",
    "gdn_chunk_fwd_gated_workspace_bytes", "gdn_chunk_bwd", "gdn_chunk_bwd_workspace_bytes", "gdn_kda_chunk_fwd",
    "gdn_kda_chunk_fwd_workspace_bytes", "gdn_chunk_fwd_varlen", "gdn_chunk_fwd_varlen_workspace_bytes",
    "gdn_chunk_fwd_scan", "gdn_chunk_fwd_scan_workspace_bytes", "gdn_chunk_fwd_scan_segments", "gdn_chunk_transport",
    "gdn_chunk_transport_workspace_bytes", "EXPORTED_SYMBOLS", "test_hooks", "gdn_chunk_fwd_noalloc",
    "debug_checks", "gdn_debug_take_flags", "gdn_debug_self_test",
    "GDN_NOALLOC_SCRATCH_BYTES",
]

GDN_F32 = 0
GDN_BF16 = 1
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/gdn.h
EXPORTED_SYMBOLS = ("gdn_chunk_fwd", "gdn_recurrent_step", "gdn_chunk_fwd_workspace_bytes",
                    "gdn_chunk_fwd_kernel_name", "gdn_status_string", "gdn_qkv_prologue",
                    "gdn_gated_rmsnorm", "gdn_chunk_fwd_gated", "gdn_chunk_fwd_gated_workspace_bytes",
                    "gdn_chunk_bwd", "gdn_chunk_bwd_workspace_bytes", "gdn_kda_chunk_fwd",
                    "gdn_kda_chunk_fwd_workspace_bytes", "gdn_chunk_fwd_varlen", "gdn_chunk_fwd_varlen_workspace_bytes",
                    "gdn_chunk_fwd_scan", "gdn_chunk_fwd_scan_workspace_bytes", "gdn_chunk_fwd_scan_segments",
                    "gdn_chunk_transport", "gdn_chunk_transport_workspace_bytes", "gdn_chunk_fwd_noalloc")

_HERE = os.path.dirname(os.path.abspath(__file__))
_libs = {}
_variant = "release"


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({gdn_status_string(status)})")


def library_path(variant: str = "release") -> str:
    """libgdn.so, or (variant "hooks") libgdn_hooks.so: the same kernels, with the automatic route
    choice open to environment overrides (GDN_MFMA_PATH, GDN_MFMA_BV, GDN_SPLIT_BV, GDN_SPLIT_PIECE,
    GDN_DISABLE_MFMA, GDN_SCAN_SEGMENTS) so that tests can run every kernel family; or (variant
    "debug") libgdn_debug.so: the hooks build whose prefill kernels also check their indices
    (include/gdn_debug.h)."""
    name = {"release": "libgdn.so", "hooks": "libgdn_hooks.so", "debug": "libgdn_debug.so"}[variant]
    return os.path.join(_HERE, name)


@contextlib.contextmanager
def test_hooks():
    """Route every call made inside the block through libgdn_hooks.so (a testing aid)."""
    global _variant
    prev = _variant
    load_library("hooks")
    _variant = "hooks"
    try:
        yield
    finally:
        _variant = prev


@contextlib.contextmanager
def debug_checks():
    """Route every call made inside the block through libgdn_debug.so (a testing aid); read its
    failed index checks with gdn_debug_take_flags()."""
    global _variant
    prev = _variant
    load_library("debug")
    _variant = "debug"
    try:
        yield
    finally:
        _variant = prev


def gdn_debug_take_flags() -> int:
    """The debug build's failed index checks since the last call (0: none), then cleared."""
    lib = load_library("debug")
    return int(lib.gdn_debug_take_flags())


def gdn_debug_self_test(bit: int) -> None:
    """Make the debug build's check at `bit` fail once (the flags' path itself under test)."""
    if load_library("debug").gdn_debug_self_test(bit) != 0:
        raise GdnError(7, "gdn_debug_self_test")


def load_library(variant: str | None = None):
    """Load libgdn.so (or the test-hooks build; raises if it has not been built)."""
    v = variant or _variant
    if v in _libs:
        return _libs[v]
    path = library_path(v)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                           "or `python gated_deltanet_linear_delta_amd/build.py`")
    lib = ctypes.CDLL(path)
    vp, fp, i, f, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gdn_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 7 + [i, f, vp, sz, vp]
    lib.gdn_chunk_fwd.restype = i
    lib.gdn_recurrent_step.argtypes = [vp, vp, vp, fp, fp, fp, vp] + [i] * 5 + [i, f, vp]
    lib.gdn_recurrent_step.restype = i
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [i] * 7 + [i]
    lib.gdn_chunk_fwd_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd_kernel_name.argtypes = [i] * 7 + [i]
    lib.gdn_chunk_fwd_kernel_name.restype = ctypes.c_char_p
    if hasattr(lib, "gdn_debug_take_flags"):
        lib.gdn_debug_take_flags.argtypes = []
        lib.gdn_debug_take_flags.restype = ctypes.c_uint
        lib.gdn_debug_self_test.argtypes = [i]
        lib.gdn_debug_self_test.restype = i
    lib.gdn_status_string.argtypes = [i]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_qkv_prologue.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, vp, vp, vp] + [i] * 7 + [i, f, vp]
    lib.gdn_qkv_prologue.restype = i
    lib.gdn_gated_rmsnorm.argtypes = [vp, vp, fp, i, vp, i, i, i, i, i, f, vp]
    lib.gdn_gated_rmsnorm.restype = i
    lib.gdn_chunk_fwd_gated.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, fp, i, f, vp] + [i] * 7 + [i, f, vp, sz, vp]
    lib.gdn_chunk_fwd_gated.restype = i
    lib.gdn_chunk_fwd_gated_workspace_bytes.argtypes = [i] * 7 + [i]
    lib.gdn_chunk_fwd_gated_workspace_bytes.restype = sz
    lib.gdn_chunk_bwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, vp, vp, fp, fp, fp] + [i] * 6 + [i, f, vp, sz, vp]
    lib.gdn_chunk_bwd.restype = i
    lib.gdn_chunk_bwd_workspace_bytes.argtypes = [i] * 6 + [i]
    lib.gdn_chunk_bwd_workspace_bytes.restype = sz
    lib.gdn_kda_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 7 + [i, f, vp, sz, vp]
    lib.gdn_kda_chunk_fwd_workspace_bytes.argtypes = [i] * 7 + [i]
    lib.gdn_kda_chunk_fwd_workspace_bytes.restype = sz
    lib.gdn_kda_chunk_fwd.restype = i
    lib.gdn_chunk_fwd_varlen.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, vp] + [i] * 8 + [i, f, vp, sz, vp]
    lib.gdn_chunk_fwd_varlen.restype = i
    lib.gdn_chunk_fwd_varlen_workspace_bytes.argtypes = [i] * 7 + [i]
    lib.gdn_chunk_fwd_varlen_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd_scan.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 7 + [i, f, i, vp, sz, vp]
    lib.gdn_chunk_fwd_scan.restype = i
    lib.gdn_chunk_fwd_scan_workspace_bytes.argtypes = [i] * 7 + [i, i]
    lib.gdn_chunk_fwd_scan_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd_scan_segments.argtypes = [i] * 7 + [i, i]
    lib.gdn_chunk_fwd_scan_segments.restype = i
    lib.gdn_chunk_transport.argtypes = [vp, vp, vp, fp, fp, fp, fp] + [i] * 7 + [i, vp, sz, vp]
    lib.gdn_chunk_transport.restype = i
    lib.gdn_chunk_transport_workspace_bytes.argtypes = [i] * 7 + [i]
    lib.gdn_chunk_transport_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 7 + [i, f, vp]
    lib.gdn_chunk_fwd_noalloc.restype = i
    _libs[v] = lib
    return lib


def gdn_status_string(status: int) -> str:
    return load_library().gdn_status_string(int(status)).decode()


def gdn_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk=64, dtype=GDN_BF16) -> int:
    return int(load_library().gdn_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype))


def gdn_chunk_fwd_gated_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk=64, dtype=GDN_BF16) -> int:
    return int(load_library().gdn_chunk_fwd_gated_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype))


def gdn_chunk_bwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, dtype=GDN_BF16) -> int:
    return int(load_library().gdn_chunk_bwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, dtype))


def gdn_chunk_fwd_varlen_workspace_bytes(N, max_seqlen, Hqk, Hv, dk, dv, chunk=64, dtype=GDN_BF16) -> int:
    return int(load_library().gdn_chunk_fwd_varlen_workspace_bytes(N, max_seqlen, Hqk, Hv, dk, dv, chunk, dtype))


def gdn_kda_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk=64, dtype=GDN_BF16) -> int:
    return int(load_library().gdn_kda_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype))


def gdn_chunk_fwd_scan_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk=64, dtype=GDN_BF16, segments=1) -> int:
    return int(load_library().gdn_chunk_fwd_scan_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype, segments))


def gdn_chunk_fwd_scan_segments(B, T, Hqk, Hv, dk, dv, chunk=64, dtype=GDN_BF16, segments=1) -> int:
    return int(load_library().gdn_chunk_fwd_scan_segments(B, T, Hqk, Hv, dk, dv, chunk, dtype, segments))


def gdn_chunk_transport_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk=64, dtype=GDN_BF16) -> int:
    return int(load_library().gdn_chunk_transport_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype))


def gdn_chunk_fwd_kernel_name(B, T, Hqk, Hv, dk, dv, chunk=64, dtype=GDN_BF16):
    r = load_library().gdn_chunk_fwd_kernel_name(B, T, Hqk, Hv, dk, dv, chunk, dtype)
    return None if r is None else r.decode()


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dense(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def gdn_chunk_fwd(q, k, v, g, beta, initial_state=None, output_final_state=True, chunk=64,
                  scale=1.0, o=None, final_state=None, workspace=None, stream=None):
    """Prefill.  q, k [B,T,Hqk,dk]; v [B,T,Hv,dv] (bf16 or f32, all alike); g, beta [B,T,Hv]
    float32; initial_state [B,Hv,dk,dv] float32 or None.  Returns (o [B,T,Hv,dv], final_state or
    None).  ``final_state`` may be passed (even as ``initial_state`` itself, for an in-place
    update); ``o`` may be passed preallocated."""
    torch = _torch()
    lib = load_library()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    _check_dense("q", q, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("k", k, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("v", v, (B, T, Hv, dv), q.dtype, dev)
    _check_dense("g", g, (B, T, Hv), torch.float32, dev)
    _check_dense("beta", beta, (B, T, Hv), torch.float32, dev)
    if initial_state is not None:
        _check_dense("initial_state", initial_state, (B, Hv, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=dev)
    _check_dense("o", o, (B, T, Hv, dv), q.dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check_dense("final_state", final_state, (B, Hv, dk, dv), torch.float32, dev)
    dt = _dtype_code(q)
    need = int(lib.gdn_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dt))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(final_state), _ptr(o), B, T, Hqk, Hv, dk, dv, int(chunk), dt,
                           float(scale), _ptr(workspace), wbytes, _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_fwd")
    return o, final_state


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, initial_state, o, final_state=None, chunk=64, scale=1.0,
                          stream=None):
    """Prefill through gdn_chunk_fwd_noalloc: as :func:`gdn_chunk_fwd`, with the workspace in the
    library's fixed per-device array.  The caller passes every output (``o``, and ``final_state``
    or None); this wrapper allocates nothing.  Returns (o, final_state)."""
    torch = _torch()
    lib = load_library()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    _check_dense("q", q, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("k", k, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("v", v, (B, T, Hv, dv), q.dtype, dev)
    _check_dense("g", g, (B, T, Hv), torch.float32, dev)
    _check_dense("beta", beta, (B, T, Hv), torch.float32, dev)
    if initial_state is not None:
        _check_dense("initial_state", initial_state, (B, Hv, dk, dv), torch.float32, dev)
    _check_dense("o", o, (B, T, Hv, dv), q.dtype, dev)
    if final_state is not None:
        _check_dense("final_state", final_state, (B, Hv, dk, dv), torch.float32, dev)
    st = lib.gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                   _ptr(final_state), _ptr(o), B, T, Hqk, Hv, dk, dv, int(chunk), _dtype_code(q),
                                   float(scale), _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_fwd_noalloc")
    return o, final_state


def gdn_recurrent_step(q, k, v, g, beta, state, scale=1.0, o=None, stream=None):
    """Decode step.  q, k [B,Hqk,dk]; v [B,Hv,dv]; g, beta [B,Hv] float32; state [B,Hv,dk,dv]
    float32, updated in place.  Returns o [B,Hv,dv]."""
    torch = _torch()
    lib = load_library()
    B, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    dev = q.device
    _check_dense("q", q, (B, Hqk, dk), q.dtype, dev)
    _check_dense("k", k, (B, Hqk, dk), q.dtype, dev)
    _check_dense("v", v, (B, Hv, dv), q.dtype, dev)
    _check_dense("g", g, (B, Hv), torch.float32, dev)
    _check_dense("beta", beta, (B, Hv), torch.float32, dev)
    _check_dense("state", state, (B, Hv, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, Hv, dv), dtype=q.dtype, device=dev)
    _check_dense("o", o, (B, Hv, dv), q.dtype, dev)
    st = lib.gdn_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                _ptr(o), B, Hqk, Hv, dk, dv, _dtype_code(q), float(scale),
                                _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_recurrent_step")
    return o


def gdn_qkv_prologue(q_in, k_in, v_in, conv_q, conv_k, conv_v, conv_state_in=None,
                     output_conv_state=False, eps=1e-6, q=None, k=None, v=None, conv_state_out=None,
                     stream=None):
    """Short causal conv, SiLU and q/k L2 norm.  q_in, k_in [B,T,Hqk,dk]; v_in [B,T,Hv,dv] (bf16
    or f32, all alike); conv_q, conv_k [Hqk*dk, W], conv_v [Hv*dv, W] float32; conv_state_in
    [B, 2*Hqk*dk + Hv*dv, W-1] float32 or None.  Returns (q, k, v, conv_state_out or None)."""
    torch = _torch()
    lib = load_library()
    B, T, Hqk, dk = q_in.shape
    Hv, dv = v_in.shape[2], v_in.shape[3]
    W = conv_q.shape[1]
    dev = q_in.device
    _check_dense("q_in", q_in, (B, T, Hqk, dk), q_in.dtype, dev)
    _check_dense("k_in", k_in, (B, T, Hqk, dk), q_in.dtype, dev)
    _check_dense("v_in", v_in, (B, T, Hv, dv), q_in.dtype, dev)
    _check_dense("conv_q", conv_q, (Hqk * dk, W), torch.float32, dev)
    _check_dense("conv_k", conv_k, (Hqk * dk, W), torch.float32, dev)
    _check_dense("conv_v", conv_v, (Hv * dv, W), torch.float32, dev)
    cs = (B, 2 * Hqk * dk + Hv * dv, W - 1)
    if conv_state_in is not None:
        _check_dense("conv_state_in", conv_state_in, cs, torch.float32, dev)
    if conv_state_out is None and output_conv_state:
        conv_state_out = torch.empty(cs, dtype=torch.float32, device=dev)
    if conv_state_out is not None:
        _check_dense("conv_state_out", conv_state_out, cs, torch.float32, dev)
    q = torch.empty_like(q_in) if q is None else q
    k = torch.empty_like(k_in) if k is None else k
    v = torch.empty_like(v_in) if v is None else v
    _check_dense("q", q, (B, T, Hqk, dk), q_in.dtype, dev)
    _check_dense("k", k, (B, T, Hqk, dk), q_in.dtype, dev)
    _check_dense("v", v, (B, T, Hv, dv), q_in.dtype, dev)
    st = lib.gdn_qkv_prologue(_ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(conv_q), _ptr(conv_k), _ptr(conv_v),
                              _ptr(conv_state_in), _ptr(conv_state_out), _ptr(q), _ptr(k), _ptr(v), B, T, Hqk,
                              Hv, dk, dv, W, _dtype_code(q_in), float(eps), _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_qkv_prologue")
    return q, k, v, conv_state_out


def gdn_gated_rmsnorm(o, z, weight, eps=1e-6, y=None, stream=None):
    """y = RMSNorm(o) * weight * silu(z) per value head.  o, z [B,T,Hv,dv] (bf16 or f32);
    weight [dv] (shared by the heads) or [Hv, dv] float32.  ``y`` may be ``o`` or ``z``."""
    torch = _torch()
    lib = load_library()
    B, T, Hv, dv = o.shape
    dev = o.device
    _check_dense("o", o, (B, T, Hv, dv), o.dtype, dev)
    _check_dense("z", z, (B, T, Hv, dv), o.dtype, dev)
    per_head = 1 if weight.dim() == 2 else 0
    _check_dense("weight", weight, (Hv, dv) if per_head else (dv,), torch.float32, dev)
    y = torch.empty_like(o) if y is None else y
    _check_dense("y", y, (B, T, Hv, dv), o.dtype, dev)
    st = lib.gdn_gated_rmsnorm(_ptr(o), _ptr(z), _ptr(weight), per_head, _ptr(y), B, T, Hv, dv,
                               _dtype_code(o), float(eps), _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_gated_rmsnorm")
    return y


def gdn_chunk_fwd_gated(q, k, v, g, beta, z, norm_weight, initial_state=None, output_final_state=True,
                        chunk=64, scale=1.0, eps=1e-6, y=None, final_state=None, workspace=None,
                        stream=None):
    """Prefill, then y = RMSNorm(o) * norm_weight * silu(z) per value head.  Arguments as
    :func:`gdn_chunk_fwd`, plus z [B,T,Hv,dv] (dtype of q) and norm_weight [dv] or [Hv, dv]
    float32.  Returns (y, final_state or None); ``y`` may be ``z``."""
    torch = _torch()
    lib = load_library()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    _check_dense("q", q, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("k", k, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("v", v, (B, T, Hv, dv), q.dtype, dev)
    _check_dense("g", g, (B, T, Hv), torch.float32, dev)
    _check_dense("beta", beta, (B, T, Hv), torch.float32, dev)
    _check_dense("z", z, (B, T, Hv, dv), q.dtype, dev)
    per_head = 1 if norm_weight.dim() == 2 else 0
    _check_dense("norm_weight", norm_weight, (Hv, dv) if per_head else (dv,), torch.float32, dev)
    if initial_state is not None:
        _check_dense("initial_state", initial_state, (B, Hv, dk, dv), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=dev)
    _check_dense("y", y, (B, T, Hv, dv), q.dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check_dense("final_state", final_state, (B, Hv, dk, dv), torch.float32, dev)
    dt = _dtype_code(q)
    need = int(lib.gdn_chunk_fwd_gated_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dt))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                 _ptr(final_state), _ptr(z), _ptr(norm_weight), per_head, float(eps), _ptr(y),
                                 B, T, Hqk, Hv, dk, dv, int(chunk), dt, float(scale), _ptr(workspace), wbytes,
                                 _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_fwd_gated")
    return y, final_state


def gdn_chunk_bwd(q, k, v, g, beta, grad_o, initial_state=None, grad_final_state=None, scale=1.0,
                  want_grad_initial_state=True, workspace=None, stream=None):
    """Backward pass of :func:`gdn_chunk_fwd`.  Inputs as that call plus grad_o [B,T,Hv,dv]
    (dtype of q) and grad_final_state [B,Hv,dk,dv] float32 or None.  Returns a dict of dq, dk
    [B,T,Hqk,dk], dv [B,T,Hv,dv] (dtype of q), dg, dbeta [B,T,Hv] float32 and ds0
    [B,Hv,dk,dv] float32 (None when not wanted)."""
    torch = _torch()
    lib = load_library()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    _check_dense("q", q, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("k", k, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("v", v, (B, T, Hv, dv), q.dtype, dev)
    _check_dense("g", g, (B, T, Hv), torch.float32, dev)
    _check_dense("beta", beta, (B, T, Hv), torch.float32, dev)
    _check_dense("grad_o", grad_o, (B, T, Hv, dv), q.dtype, dev)
    if initial_state is not None:
        _check_dense("initial_state", initial_state, (B, Hv, dk, dv), torch.float32, dev)
    if grad_final_state is not None:
        _check_dense("grad_final_state", grad_final_state, (B, Hv, dk, dv), torch.float32, dev)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dg=torch.empty_like(g), dbeta=torch.empty_like(beta),
               ds0=torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev) if want_grad_initial_state else None)
    dt = _dtype_code(q)
    need = int(lib.gdn_chunk_bwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, dt))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(grad_o),
                           _ptr(grad_final_state), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                           _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["ds0"]), B, T, Hqk, Hv, dk, dv, dt,
                           float(scale), _ptr(workspace), wbytes, _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_bwd")
    return out


def gdn_kda_chunk_fwd(q, k, v, g, beta, initial_state=None, output_final_state=True, chunk=None, scale=1.0,
                      o=None, final_state=None, workspace=None, stream=None):
    """Kimi Delta Attention prefill.  q, k [B,T,Hqk,dk]; v [B,T,Hv,dv] (bf16 or f32, all alike);
    g [B,T,Hv,dk] float32 (log decay per key channel); beta [B,T,Hv] float32; initial_state
    [B,Hv,dk,dv] float32 or None.  chunk 64 runs the matrix-core kernels (bf16, head dims 64 or
    128), 16 or 32 the float32 vector kernel; None picks 64 where it applies, else 32.  Returns
    (o [B,T,Hv,dv], final_state or None)."""
    torch = _torch()
    lib = load_library()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    _check_dense("q", q, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("k", k, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("v", v, (B, T, Hv, dv), q.dtype, dev)
    _check_dense("g", g, (B, T, Hv, dk), torch.float32, dev)
    _check_dense("beta", beta, (B, T, Hv), torch.float32, dev)
    if initial_state is not None:
        _check_dense("initial_state", initial_state, (B, Hv, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=dev)
    _check_dense("o", o, (B, T, Hv, dv), q.dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check_dense("final_state", final_state, (B, Hv, dk, dv), torch.float32, dev)
    dt = _dtype_code(q)
    if chunk is None:
        chunk = 64 if (dt == GDN_BF16 and dk in (64, 128) and dv in (64, 128)) else 32
    need = int(lib.gdn_kda_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, int(chunk), dt))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                               _ptr(final_state), _ptr(o), B, T, Hqk, Hv, dk, dv, int(chunk), dt,
                               float(scale), _ptr(workspace), wbytes, _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_kda_chunk_fwd")
    return o, final_state


def gdn_chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, max_seqlen, initial_state=None, output_final_state=True,
                         chunk=64, scale=1.0, o=None, final_state=None, workspace=None, stream=None):
    """Prefill of packed sequences.  q, k [total_T, Hqk, dk]; v [total_T, Hv, dv]; g, beta
    [total_T, Hv] float32; cu_seqlens int32 [N+1] on the device (offsets, non-decreasing from 0 to
    total_T); max_seqlen the longest sequence (an int the caller knows); initial_state
    [N, Hv, dk, dv] float32 or None.  Returns (o [total_T, Hv, dv], final_state or None)."""
    torch = _torch()
    lib = load_library()
    total, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    dev = q.device
    N = cu_seqlens.numel() - 1
    _check_dense("q", q, (total, Hqk, dk), q.dtype, dev)
    _check_dense("k", k, (total, Hqk, dk), q.dtype, dev)
    _check_dense("v", v, (total, Hv, dv), q.dtype, dev)
    _check_dense("g", g, (total, Hv), torch.float32, dev)
    _check_dense("beta", beta, (total, Hv), torch.float32, dev)
    _check_dense("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    if initial_state is not None:
        _check_dense("initial_state", initial_state, (N, Hv, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((total, Hv, dv), dtype=q.dtype, device=dev)
    _check_dense("o", o, (total, Hv, dv), q.dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check_dense("final_state", final_state, (N, Hv, dk, dv), torch.float32, dev)
    dt = _dtype_code(q)
    need = int(lib.gdn_chunk_fwd_varlen_workspace_bytes(N, int(max_seqlen), Hqk, Hv, dk, dv, int(chunk), dt))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                  _ptr(final_state), _ptr(o), _ptr(cu_seqlens), N, int(max_seqlen), total, Hqk, Hv,
                                  dk, dv, int(chunk), dt, float(scale), _ptr(workspace), wbytes, _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_fwd_varlen")
    return o, final_state


def gdn_chunk_fwd_scan(q, k, v, g, beta, initial_state=None, output_final_state=True, chunk=64, scale=1.0,
                       segments=4, o=None, final_state=None, workspace=None, stream=None):
    """Prefill with each (batch, value head) chain cut into ``segments`` segments (the affine
    chunk scan).  Arguments and results as :func:`gdn_chunk_fwd` (bf16, chunk 64, head dims 64 or
    128)."""
    torch = _torch()
    lib = load_library()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    _check_dense("q", q, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("k", k, (B, T, Hqk, dk), q.dtype, dev)
    _check_dense("v", v, (B, T, Hv, dv), q.dtype, dev)
    _check_dense("g", g, (B, T, Hv), torch.float32, dev)
    _check_dense("beta", beta, (B, T, Hv), torch.float32, dev)
    if initial_state is not None:
        _check_dense("initial_state", initial_state, (B, Hv, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=dev)
    _check_dense("o", o, (B, T, Hv, dv), q.dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check_dense("final_state", final_state, (B, Hv, dk, dv), torch.float32, dev)
    dt = _dtype_code(q)
    need = int(lib.gdn_chunk_fwd_scan_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dt, int(segments)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_chunk_fwd_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                _ptr(final_state), _ptr(o), B, T, Hqk, Hv, dk, dv, int(chunk), dt, float(scale),
                                int(segments), _ptr(workspace), wbytes, _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_fwd_scan")
    return o, final_state


def gdn_chunk_transport(k, v, g, beta, q=None, chunk=64, m_out=None, n_out=None, workspace=None, stream=None):
    """The affine state map of the given tokens per (batch, value head): after them the stored
    state is M h + N for entry state h.  k [B,T,Hqk,dk], v [B,T,Hv,dv] bf16; g, beta [B,T,Hv]
    float32; q optional (the map does not depend on it).  Returns (M [B,Hv,dk,dk], N [B,Hv,dk,dv])
    float32."""
    torch = _torch()
    lib = load_library()
    B, T, Hqk, dk = k.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = k.device
    if q is not None:
        _check_dense("q", q, (B, T, Hqk, dk), k.dtype, dev)
    _check_dense("k", k, (B, T, Hqk, dk), k.dtype, dev)
    _check_dense("v", v, (B, T, Hv, dv), k.dtype, dev)
    _check_dense("g", g, (B, T, Hv), torch.float32, dev)
    _check_dense("beta", beta, (B, T, Hv), torch.float32, dev)
    if m_out is None:
        m_out = torch.empty((B, Hv, dk, dk), dtype=torch.float32, device=dev)
    if n_out is None:
        n_out = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    _check_dense("m_out", m_out, (B, Hv, dk, dk), torch.float32, dev)
    _check_dense("n_out", n_out, (B, Hv, dk, dv), torch.float32, dev)
    dt = _dtype_code(k)
    need = int(lib.gdn_chunk_transport_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dt))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_chunk_transport(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(m_out), _ptr(n_out), B, T,
                                 Hqk, Hv, dk, dv, int(chunk), dt, _ptr(workspace), wbytes, _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_transport")
    return m_out, n_out
