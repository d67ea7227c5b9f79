"""Python binding of libssm (include/ssm.h): selective-scan and scalar-decay
chunked-SSD forward on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libssm.so``.  PyTorch supplies device memory and the current HIP
stream.  If ``libssm.so`` is missing the calls raise; there is no fallback.

    from state_space_model_ssm_amd import scan_fwd, ssd_chunked_fwd
    y, h_last = scan_fwd(u, delta, A, B, C, D, z)
    y, h_last = ssd_chunked_fwd(x, dt, A, B, C, D)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "SSM_F32", "SSM_BF16", "SSM_DT_SOFTPLUS", "SSM_LAM_SIGMOID", "SsmError", "ScanDims", "SsdDims", "lib", "library_path",
    "scan_fwd", "scan_fwd_noalloc", "scan_bwd", "ssd_chunked_fwd", "ssd_trap_chunked_fwd", "ssd_rope_chunked_fwd",
    "ssd_rope_trap_chunked_fwd", "scan_step", "ssd_step",
    "ssd_trap_step", "ssd_bwd", "ssd_bwd_workspace_size",
    "rope_bc", "rope_bc_bwd", "rope_bc_bwd_workspace_size", "RopeDims",
    "scan_workspace_size",
    "scan_resolved_chunks", "ssd_workspace_size", "status_string", "last_error", "version",
]

SSM_F32, SSM_BF16 = 0, 1
SSM_DT_SOFTPLUS, SSM_LAM_SIGMOID = 1, 2   # dims.flags bits (Phase-0 maps of dt and lam)
STATUS = {0: "SSM_OK", -1: "SSM_ERR_NULL", -2: "SSM_ERR_SHAPE", -3: "SSM_ERR_DTYPE",
          -4: "SSM_ERR_ALIGN", -5: "SSM_ERR_UNSUPPORTED", -6: "SSM_ERR_WORKSPACE",
          -7: "SSM_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssm.so")
_lib = None


class SsmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class ScanDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("seqlen", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("n_chunks", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("dt_bias", ctypes.c_void_p)]


class SsdDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("dt_bias", ctypes.c_void_p)]


class StepDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32), ("dt_bias", ctypes.c_void_p)]


class SsdStepDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("dt_bias", ctypes.c_void_p)]


class RopeDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64), ("theta_heads", ctypes.c_int64),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("dt_bias", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libssm (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m state_space_model_ssm_amd.build` "
                "(hipcc, gfx950). There is no fallback implementation.")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        L.ssm_scan_fwd.argtypes = [vp] * 10 + [ctypes.POINTER(ScanDims), vp]
        L.ssm_scan_fwd.restype = i32
        L.ssm_scan_fwd_noalloc.argtypes = [vp] * 10 + [ctypes.POINTER(ScanDims), vp]
        L.ssm_scan_fwd_noalloc.restype = i32
        L.ssm_scan_workspace_size.argtypes = [ctypes.POINTER(ScanDims), ctypes.POINTER(ctypes.c_size_t)]
        L.ssm_scan_workspace_size.restype = i32
        L.ssm_scan_resolved_chunks.argtypes = [ctypes.POINTER(ScanDims), ctypes.POINTER(ctypes.c_int32)]
        L.ssm_scan_resolved_chunks.restype = i32
        L.ssd_chunked_fwd.argtypes = [vp] * 10 + [ctypes.POINTER(SsdDims), vp]
        L.ssd_trap_chunked_fwd.argtypes = [vp] * 13 + [ctypes.POINTER(SsdDims), vp]
        L.ssd_trap_chunked_fwd.restype = ctypes.c_int
        i64 = ctypes.c_int64
        L.ssd_rope_chunked_fwd.argtypes = [vp] * 6 + [i64] + [vp] * 8 + [ctypes.POINTER(SsdDims), vp]
        L.ssd_rope_chunked_fwd.restype = i32
        L.ssd_rope_trap_chunked_fwd.argtypes = [vp] * 7 + [i64] + [vp] * 10 + [ctypes.POINTER(SsdDims), vp]
        L.ssd_rope_trap_chunked_fwd.restype = i32
        L.ssd_chunked_fwd.restype = i32
        L.ssd_workspace_size.argtypes = [ctypes.POINTER(SsdDims), ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_workspace_size.restype = i32
        L.ssd_bwd_workspace_size.argtypes = [ctypes.POINTER(SsdDims), ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_bwd_workspace_size.restype = i32
        L.ssd_bwd.argtypes = [vp] * 18 + [ctypes.POINTER(SsdDims), vp]
        L.ssd_bwd.restype = i32
        L.ssd_trap_bwd.argtypes = [vp] * 24 + [ctypes.POINTER(SsdDims), vp]
        L.ssd_trap_bwd.restype = i32
        L.ssm_scan_bwd.argtypes = [vp] * 18 + [ctypes.POINTER(ScanDims), vp]
        L.ssm_scan_bwd.restype = i32
        L.ssm_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(ScanDims), ctypes.POINTER(ctypes.c_size_t)]
        L.ssm_scan_bwd_workspace_size.restype = i32
        L.ssm_scan_step.argtypes = [vp] * 9 + [ctypes.POINTER(StepDims), vp]
        L.ssm_scan_step.restype = i32
        L.ssd_step.argtypes = [vp] * 9 + [ctypes.POINTER(SsdStepDims), vp]
        L.ssd_step.restype = i32
        L.ssd_trap_step.argtypes = [vp] * 12 + [ctypes.POINTER(SsdStepDims), vp]
        L.ssd_trap_step.restype = i32
        L.ssm_rope_bc.argtypes = [vp] * 8 + [ctypes.POINTER(RopeDims), vp]
        L.ssm_rope_bc.restype = i32
        L.ssm_rope_bc_bwd_workspace_size.argtypes = [ctypes.POINTER(RopeDims), ctypes.POINTER(ctypes.c_size_t)]
        L.ssm_rope_bc_bwd_workspace_size.restype = i32
        L.ssm_rope_bc_bwd.argtypes = [vp] * 14 + [ctypes.c_size_t, ctypes.POINTER(RopeDims), vp]
        L.ssm_rope_bc_bwd.restype = i32
        L.ssm_status_string.argtypes = [i32]
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_last_error.argtypes = []
        L.ssm_last_error.restype = ctypes.c_char_p
        L.ssm_version.argtypes = []
        L.ssm_version.restype = i32
        L.ssm_scan_workspace_bytes.argtypes = [ctypes.POINTER(ScanDims)]
        L.ssm_scan_workspace_bytes.restype = ctypes.c_size_t
        L.ssd_workspace_bytes.argtypes = [ctypes.POINTER(SsdDims)]
        L.ssd_workspace_bytes.restype = ctypes.c_size_t
        L.ssm_last_error_message.argtypes = []
        L.ssm_last_error_message.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ssm_status_string(status).decode()


def last_error() -> str:
    return lib().ssm_last_error().decode()


def version() -> int:
    return lib().ssm_version()


def _check(rc: int):
    if rc != 0:
        raise SsmError(rc, last_error())


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.float32:
        return SSM_F32
    if t == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() or None


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def _alloc_on(stream):
    """Context in which the binding allocates outputs and workspace: on the
    stream the kernels will run on.  PyTorch's caching allocator ties a block
    to the stream current at its allocation, so a workspace freed when the
    call returns is reused only by later work on that same stream, which runs
    after the kernels that still read it."""
    import contextlib
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def _out(t, shape, dtype, like, name):
    """A caller-given output tensor, checked against the shape and dtype the
    call writes (the library trusts the sizes in the dims), or a new one."""
    if t is None:
        return _torch().empty(shape, dtype=dtype, device=like.device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != like.device:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)} on {like.device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _phase0(dims, n: int, dt_softplus: bool, dt_bias, lam_sigmoid: bool = False):
    """Set the Phase-0 flags of ``dims``: softplus(dt + dt_bias) as the step
    (dt_bias: (n,) float32 or None) and sigmoid(lam) for the trapezoid."""
    if dt_bias is not None:
        if not dt_softplus:
            raise ValueError("dt_bias is used only with dt_softplus=True")
        if dt_bias.dtype != _torch().float32 or tuple(dt_bias.shape) != (n,):
            raise ValueError(f"dt_bias must be float32 of shape ({n},)")
    dims.flags = (SSM_DT_SOFTPLUS if dt_softplus else 0) | (SSM_LAM_SIGMOID if lam_sigmoid else 0)
    dims.dt_bias = _ptr(dt_bias)


def _scan_dims(u, B, in_dtype, out_dtype, n_chunks) -> ScanDims:
    batch, dim, L = u.shape
    G, N = B.shape[1], B.shape[2]
    return ScanDims(batch=batch, dim=dim, dstate=N, seqlen=L, ngroups=G, in_dtype=in_dtype,
                    out_dtype=out_dtype, n_chunks=n_chunks, flags=0, workspace=None,
                    workspace_bytes=0)


def scan_workspace_size(dims: ScanDims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ssm_scan_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def scan_resolved_chunks(dims: ScanDims) -> int:
    n = ctypes.c_int32(0)
    _check(lib().ssm_scan_resolved_chunks(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def scan_fwd(u, delta, A, B, C, D=None, z=None, *, h0=None, out_dtype=None, n_chunks: int = 0,
             return_h_last: bool = True, y=None, h_last=None, workspace=None, stream=None,
             dt_softplus: bool = False, dt_bias=None):
    """Selective-scan forward (``ssm_scan_fwd``). Returns ``(y, h_last)``.

    u, delta, z: (batch, dim, L); A: (dim, N) float32; B, C: (batch, G, N, L);
    D: (dim,) float32; h0: (batch, dim, N) float32 initial state (zero when
    None).  u/delta/B/C/z share one dtype (float32 or bfloat16); y defaults to
    that dtype, h_last is float32 (batch, dim, N) and may be h0 itself.
    dt_softplus: delta is raw and the step is softplus(delta + dt_bias)
    (dt_bias: (dim,) float32 or None).
    """
    torch = _torch()
    in_code = _dtype_code(u.dtype)
    out_dt = u.dtype if out_dtype is None else out_dtype
    out_code = _dtype_code(out_dt)
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z)):
        if t is not None and t.dtype != u.dtype:
            raise TypeError(f"{name} must have dtype {u.dtype}")
    for name, t in (("A", A), ("D", D)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    batch, dim, L = u.shape
    N = B.shape[2]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("delta and z must have the shape of u")
    if B.dim() != 4 or B.shape[0] != batch or B.shape[3] != L or C.shape != B.shape:
        raise ValueError("B and C must be (batch, ngroups, dstate, seqlen)")
    if A.shape != (dim, N) or (D is not None and D.shape != (dim,)):
        raise ValueError("A must be (dim, dstate) and D (dim,)")
    if h0 is not None and (h0.dtype != torch.float32 or h0.shape != (batch, dim, N)):
        raise ValueError("h0 must be float32 (batch, dim, dstate)")
    dims = _scan_dims(u, B, in_code, out_code, n_chunks)
    _phase0(dims, dim, dt_softplus, dt_bias)
    need = scan_workspace_size(dims)
    with _alloc_on(stream):
        y = _out(y, (batch, dim, L), out_dt, u, "y")
        if h_last is not None or return_h_last:
            h_last = _out(h_last, (batch, dim, N), torch.float32, u, "h_last")
        if need > 0:
            if workspace is None or workspace.numel() * workspace.element_size() < need:
                workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
            dims.workspace = _ptr(workspace)
            dims.workspace_bytes = workspace.numel() * workspace.element_size()
    rc = lib().ssm_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                            _ptr(h0), _ptr(y), _ptr(h_last), ctypes.byref(dims), _stream(stream))
    _check(rc)
    return y, h_last


def scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, *, y, h_last=None, h0=None, n_chunks: int = 0,
                     stream=None, dt_softplus: bool = False, dt_bias=None):
    """Selective-scan forward through ``ssm_scan_fwd_noalloc``: the library's
    static scratch holds the chunked carry, so the call allocates nothing.
    The caller passes y (and h_last, if wanted) preallocated; arguments are
    otherwise those of ``scan_fwd``.  Returns ``(y, h_last)``."""
    torch = _torch()
    in_code = _dtype_code(u.dtype)
    out_code = _dtype_code(y.dtype)
    batch, dim, L = u.shape
    N = B.shape[2]
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z)):
        if t is not None and t.dtype != u.dtype:
            raise TypeError(f"{name} must have dtype {u.dtype}")
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("delta and z must have the shape of u")
    if B.dim() != 4 or B.shape[0] != batch or B.shape[3] != L or C.shape != B.shape:
        raise ValueError("B and C must be (batch, ngroups, dstate, seqlen)")
    if A.shape != (dim, N) or A.dtype != torch.float32 or (D is not None and (D.shape != (dim,) or
                                                                             D.dtype != torch.float32)):
        raise ValueError("A must be float32 (dim, dstate) and D float32 (dim,)")
    if h0 is not None and (h0.dtype != torch.float32 or h0.shape != (batch, dim, N)):
        raise ValueError("h0 must be float32 (batch, dim, dstate)")
    _out(y, (batch, dim, L), y.dtype, u, "y")
    if h_last is not None:
        _out(h_last, (batch, dim, N), torch.float32, u, "h_last")
    dims = _scan_dims(u, B, in_code, out_code, n_chunks)
    _phase0(dims, dim, dt_softplus, dt_bias)
    _check(lib().ssm_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(h0), _ptr(y), _ptr(h_last), ctypes.byref(dims), _stream(stream)))
    return y, h_last


def scan_bwd_workspace_size(dims: ScanDims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ssm_scan_bwd_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def scan_bwd(u, delta, A, B, C, D=None, z=None, *, dy, h0=None, dh_last=None, workspace=None, stream=None,
             dt_softplus: bool = False, dt_bias=None):
    """Selective-scan backward (``ssm_scan_bwd``): gradients of a loss with
    upstream gradients dy (shaped like y, in y's dtype) and dh_last (float32,
    optional).  Returns a dict du, ddelta (u's dtype), dA, dB, dC (float32),
    dD (float32, when D is given), dz (u's dtype, when z is given) and dh0
    (float32).  With dt_softplus, ddelta is the gradient of the raw delta
    (that of dt_bias is its sum over batch and steps)."""
    torch = _torch()
    in_code = _dtype_code(u.dtype)
    out_code = _dtype_code(dy.dtype)
    batch, dim, L = u.shape
    G, N = B.shape[1], B.shape[2]
    if dy.shape != u.shape or (dh_last is not None and dh_last.shape != (batch, dim, N)):
        raise ValueError("dy must be shaped like u and dh_last (batch, dim, dstate)")
    if h0 is not None and (h0.dtype != torch.float32 or h0.shape != (batch, dim, N)):
        raise ValueError("h0 must be float32 (batch, dim, dstate)")
    dims = _scan_dims(u, B, in_code, out_code, 0)
    _phase0(dims, dim, dt_softplus, dt_bias)
    need = scan_bwd_workspace_size(dims)
    f32 = torch.float32
    with _alloc_on(stream):
        if need > 0:
            if workspace is None or workspace.numel() * workspace.element_size() < need:
                workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
            dims.workspace = _ptr(workspace)
            dims.workspace_bytes = workspace.numel() * workspace.element_size()
        g = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u),
             "dA": torch.empty((dim, N), dtype=f32, device=u.device),
             "dB": torch.empty(B.shape, dtype=f32, device=u.device),
             "dC": torch.empty(C.shape, dtype=f32, device=u.device),
             "dD": None if D is None else torch.empty((dim,), dtype=f32, device=u.device),
             "dz": None if z is None else torch.empty_like(u),
             "dh0": torch.empty((batch, dim, N), dtype=f32, device=u.device)}
    _check(lib().ssm_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                              _ptr(dy), _ptr(dh_last), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                              _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]),
                              ctypes.byref(dims), _stream(stream)))
    return g


def _ssd_dims(x, B, chunk, in_dtype, out_dtype) -> SsdDims:
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return SsdDims(batch=batch, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G, chunk=chunk,
                   in_dtype=in_dtype, out_dtype=out_dtype, flags=0, reserved=0, workspace=None,
                   workspace_bytes=0)


def ssd_workspace_size(dims: SsdDims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ssd_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def _ssd_call(x, dt, lam, A, B, C, D=None, z=None, *, h0=None, chunk: int = 64, out_dtype=None,
                    return_h_last: bool = True, y=None, h_last=None, stream=None,
                    dt_softplus: bool = False, dt_bias=None, lam_sigmoid: bool = False,
                    x_prev=None, B_prev=None, rope=None):
    """Scalar-decay chunked SSD forward, plain (lam None: ``ssd_chunked_fwd``)
    or trapezoidal (``ssd_trap_chunked_fwd``). Returns ``(y, h_last)``.
    With ``rope`` (a dict: theta, angle0, angle_last, return_angle_last,
    B_last, return_B_last) the fused rotary forms ``ssd_rope_chunked_fwd`` /
    ``ssd_rope_trap_chunked_fwd``; returns ``(y, h_last, angle_last, B_last)``.

    x, z: (batch, L, H, P) bf16; dt: (batch, L, H) bf16; A, D: (H,) float32;
    B, C: (batch, L, G, N) bf16; h0: (batch, H, P, N) float32 initial state
    (zero when None).  h_last is float32 (batch, H, P, N) and may be h0 itself.
    """
    torch = _torch()
    in_code = _dtype_code(x.dtype)
    out_dt = x.dtype if out_dtype is None else out_dtype
    out_code = _dtype_code(out_dt)
    for name, t in (("dt", dt), ("B", B), ("C", C), ("z", z)):
        if t is not None and t.dtype != x.dtype:
            raise TypeError(f"{name} must have dtype {x.dtype}")
    for name, t in (("A", A), ("D", D)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    batch, L, H, P = x.shape
    N = B.shape[3]
    if dt.shape != (batch, L, H) or (z is not None and z.shape != x.shape):
        raise ValueError("dt must be (batch, L, H) and z shaped like x")
    if lam is not None and (lam.shape != dt.shape or lam.dtype != x.dtype):
        raise ValueError("lam must be shaped and typed like dt")
    if B.dim() != 4 or B.shape[:2] != (batch, L) or C.shape != B.shape:
        raise ValueError("B and C must be (batch, seqlen, ngroups, dstate)")
    if A.shape != (H,) or (D is not None and D.shape != (H,)):
        raise ValueError("A and D must be (nheads,)")
    if h0 is not None and (h0.dtype != torch.float32 or h0.shape != (batch, H, P, N)):
        raise ValueError("h0 must be float32 (batch, nheads, headdim, dstate)")
    if (x_prev is None) != (B_prev is None):
        raise ValueError("x_prev and B_prev are given together or not at all")
    if x_prev is not None:
        if lam is None:
            raise ValueError("x_prev and B_prev belong to the trapezoidal form")
        G = H if rope is not None else B.shape[2]  # the rotary forms take the rotated B per head
        if x_prev.shape != (batch, H, P) or B_prev.shape != (batch, G, N) or x_prev.dtype != x.dtype or \
                B_prev.dtype != x.dtype:
            raise ValueError("x_prev must be (batch, nheads, headdim) and B_prev (batch, %s, dstate), "
                             "in the dtype of x" % ("nheads" if rope is not None else "ngroups"))
    dims = _ssd_dims(x, B, chunk, in_code, out_code)
    _phase0(dims, H, dt_softplus, dt_bias, lam_sigmoid)
    if rope is not None:
        theta = rope["theta"]
        TH = theta.shape[2] if theta.dim() == 4 else -1
        if theta.dtype != x.dtype or theta.shape != (batch, L, TH, N // 2) or TH not in (1, H):
            raise ValueError("theta must be (batch, L, 1 or nheads, dstate / 2) in the dtype of x")
        angle0 = rope.get("angle0")
        if angle0 is not None and (angle0.dtype != torch.float32 or angle0.shape != (batch, H, N // 2)):
            raise ValueError("angle0 must be float32 (batch, nheads, dstate / 2)")
    with _alloc_on(stream):
        y = _out(y, (batch, L, H, P), out_dt, x, "y")
        if h_last is not None or return_h_last:
            h_last = _out(h_last, (batch, H, P, N), torch.float32, x, "h_last")
        if rope is not None:
            angle_last, B_last = rope.get("angle_last"), rope.get("B_last")
            if angle_last is not None or rope.get("return_angle_last", True):
                angle_last = _out(angle_last, (batch, H, N // 2), torch.float32, x, "angle_last")
            if B_last is not None or rope.get("return_B_last", False):
                B_last = _out(B_last, (batch, H, N), x.dtype, x, "B_last")
    if rope is not None:
        if lam is None:
            rc = lib().ssd_rope_chunked_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(theta), TH,
                                            _ptr(angle0), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last),
                                            _ptr(angle_last), _ptr(B_last), ctypes.byref(dims), _stream(stream))
        else:
            rc = lib().ssd_rope_trap_chunked_fwd(_ptr(x), _ptr(dt), _ptr(lam), _ptr(A), _ptr(B), _ptr(C),
                                                 _ptr(theta), TH, _ptr(angle0), _ptr(D), _ptr(z), _ptr(h0),
                                                 _ptr(x_prev), _ptr(B_prev), _ptr(y), _ptr(h_last),
                                                 _ptr(angle_last), _ptr(B_last), ctypes.byref(dims),
                                                 _stream(stream))
        _check(rc)
        return y, h_last, angle_last, B_last
    if lam is None:
        rc = lib().ssd_chunked_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                   _ptr(h0), _ptr(y), _ptr(h_last), ctypes.byref(dims), _stream(stream))
    else:
        rc = lib().ssd_trap_chunked_fwd(_ptr(x), _ptr(dt), _ptr(lam), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                        _ptr(z), _ptr(h0), _ptr(x_prev), _ptr(B_prev), _ptr(y), _ptr(h_last),
                                        ctypes.byref(dims), _stream(stream))
    _check(rc)
    return y, h_last


def ssd_bwd_workspace_size(dims: SsdDims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ssd_bwd_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def ssd_bwd(x, dt, A, B, C, D=None, z=None, *, dy, h0=None, dh_last=None, workspace=None, stream=None,
            dt_softplus: bool = False, dt_bias=None):
    """Scalar-decay SSD backward (``ssd_bwd``): gradients of a loss with
    upstream gradients dy (shaped like x, in the forward's output dtype) and
    dh_last (float32, optional).  Returns a dict dx, ddt, dz (bf16; dz when z is
    given), dA, dB, dC, dD (float32; dD when D is given) and dh0 (float32).
    With dt_softplus, ddt is the gradient of the raw dt."""
    return _ssd_bwd_call(x, dt, None, A, B, C, D, z, dy=dy, h0=h0, dh_last=dh_last, workspace=workspace,
                         stream=stream, dt_softplus=dt_softplus, dt_bias=dt_bias)


def ssd_trap_bwd(x, dt, lam, A, B, C, D=None, z=None, *, dy, h0=None, dh_last=None, x_prev=None, B_prev=None,
                 workspace=None, stream=None, dt_softplus: bool = False, dt_bias=None, lam_sigmoid: bool = False):
    """Trapezoidal SSD backward (``ssd_trap_bwd``): as ``ssd_bwd`` plus dlam
    (bf16) and, with x_prev and B_prev, dx_prev (bf16) and dB_prev (float32).
    With lam_sigmoid, dlam is the gradient of the raw lam."""
    return _ssd_bwd_call(x, dt, lam, A, B, C, D, z, dy=dy, h0=h0, dh_last=dh_last, workspace=workspace,
                         stream=stream, dt_softplus=dt_softplus, dt_bias=dt_bias, lam_sigmoid=lam_sigmoid,
                         x_prev=x_prev, B_prev=B_prev)


def _ssd_bwd_call(x, dt, lam, A, B, C, D, z, *, dy, h0, dh_last, workspace, stream, dt_softplus, dt_bias,
                  lam_sigmoid=False, x_prev=None, B_prev=None):
    torch = _torch()
    in_code = _dtype_code(x.dtype)
    out_code = _dtype_code(dy.dtype)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if dy.shape != x.shape or (z is not None and z.shape != x.shape) or dt.shape != (batch, L, H):
        raise ValueError("dy and z must be shaped like x, dt (batch, L, H)")
    if lam is not None and lam.shape != dt.shape:
        raise ValueError("lam must be shaped like dt")
    if B.shape != (batch, L, G, N) or C.shape != B.shape or A.shape != (H,) or (D is not None and D.shape != (H,)):
        raise ValueError("B, C must be (batch, L, ngroups, dstate) and A, D (nheads,)")
    for name, t in (("h0", h0), ("dh_last", dh_last)):
        if t is not None and (t.dtype != torch.float32 or t.shape != (batch, H, P, N)):
            raise ValueError(f"{name} must be float32 (batch, nheads, headdim, dstate)")
    if (x_prev is None) != (B_prev is None):
        raise ValueError("x_prev and B_prev are given together or not at all")
    if x_prev is not None and (x_prev.shape != (batch, H, P) or B_prev.shape != (batch, G, N)):
        raise ValueError("x_prev must be (batch, nheads, headdim) and B_prev (batch, ngroups, dstate)")
    dims = _ssd_dims(x, B, 64, in_code, out_code)
    _phase0(dims, H, dt_softplus, dt_bias, lam_sigmoid)
    need = ssd_bwd_workspace_size(dims)
    f32 = torch.float32
    with _alloc_on(stream):
        if need > 0:
            if workspace is None or workspace.numel() * workspace.element_size() < need:
                workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
            dims.workspace = _ptr(workspace)
            dims.workspace_bytes = workspace.numel() * workspace.element_size()
        g = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt),
             "dA": torch.empty((H,), dtype=f32, device=x.device),
             "dB": torch.empty(B.shape, dtype=f32, device=x.device),
             "dC": torch.empty(C.shape, dtype=f32, device=x.device),
             "dD": None if D is None else torch.empty((H,), dtype=f32, device=x.device),
             "dz": None if z is None else torch.empty_like(x),
             "dh0": torch.empty((batch, H, P, N), dtype=f32, device=x.device)}
        if lam is not None:
            g["dlam"] = torch.empty_like(lam)
            g["dx_prev"] = None if x_prev is None else torch.empty_like(x_prev)
            g["dB_prev"] = None if B_prev is None else torch.empty((batch, G, N), dtype=f32, device=x.device)
    if lam is None:
        _check(lib().ssd_bwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dy),
                             _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddt"]), _ptr(g["dA"]), _ptr(g["dB"]),
                             _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]), ctypes.byref(dims),
                             _stream(stream)))
    else:
        _check(lib().ssd_trap_bwd(_ptr(x), _ptr(dt), _ptr(lam), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                  _ptr(h0), _ptr(x_prev), _ptr(B_prev), _ptr(dy), _ptr(dh_last), _ptr(g["dx"]),
                                  _ptr(g["ddt"]), _ptr(g["dlam"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                                  _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]), _ptr(g["dx_prev"]),
                                  _ptr(g["dB_prev"]), ctypes.byref(dims), _stream(stream)))
    return g


def ssd_chunked_fwd(x, dt, A, B, C, D=None, z=None, **kw):
    """Scalar-decay chunked SSD forward (``ssd_chunked_fwd``). Returns ``(y, h_last)``.

    x, z: (batch, L, H, P) bf16; dt: (batch, L, H) bf16; A, D: (H,) float32;
    B, C: (batch, L, G, N) bf16; h0: (batch, H, P, N) float32 initial state
    (zero when None).  h_last is float32 (batch, H, P, N) and may be h0 itself.
    Keywords: h0, chunk, out_dtype, return_h_last, y, h_last, stream,
    dt_softplus (dt is raw, the step is softplus(dt + dt_bias)), dt_bias
    ((H,) float32).
    """
    return _ssd_call(x, dt, None, A, B, C, D, z, **kw)


def ssd_trap_chunked_fwd(x, dt, lam, A, B, C, D=None, z=None, **kw):
    """Trapezoidal (Mamba-3 SISO) chunked SSD (``ssd_trap_chunked_fwd``):
    lam (batch, L, H) bf16 in [0, 1] (after its sigmoid; raw with
    lam_sigmoid=True).  Keywords x_prev (batch, H, P) and B_prev (batch, G, N):
    the token before the sequence, when the call continues one.  Otherwise as
    ``ssd_chunked_fwd``. Returns ``(y, h_last)``."""
    return _ssd_call(x, dt, lam, A, B, C, D, z, **kw)


def ssd_rope_chunked_fwd(x, dt, A, B, C, theta, D=None, z=None, *, angle0=None, angle_last=None,
                         return_angle_last: bool = True, B_last=None, return_B_last: bool = False, **kw):
    """The SSD with the rotary step on B and C fused in
    (``ssd_rope_chunked_fwd``): ``rope_bc`` then ``ssd_chunked_fwd`` on the
    per-head rotated B and C, which are never stored.  theta: (batch, L, TH,
    N / 2) bf16 with TH 1 or H; angle0, angle_last: (batch, H, N / 2) float32
    (angle_last may be angle0, updated in place); B_last: (batch, H, N) bf16,
    the last step's rotated B.  Other arguments as ``ssd_chunked_fwd``.
    Returns ``(y, h_last, angle_last, B_last)`` (None for what was not asked for)."""
    rope = {"theta": theta, "angle0": angle0, "angle_last": angle_last, "return_angle_last": return_angle_last,
            "B_last": B_last, "return_B_last": return_B_last}
    return _ssd_call(x, dt, None, A, B, C, D, z, rope=rope, **kw)


def ssd_rope_trap_chunked_fwd(x, dt, lam, A, B, C, theta, D=None, z=None, *, angle0=None, angle_last=None,
                              return_angle_last: bool = True, B_last=None, return_B_last: bool = False, **kw):
    """The trapezoidal form of ``ssd_rope_chunked_fwd``
    (``ssd_rope_trap_chunked_fwd``): x_prev (batch, H, P) and B_prev (batch, H,
    N, the previous token's rotated B, e.g. the B_last of the call before).
    Returns ``(y, h_last, angle_last, B_last)``."""
    rope = {"theta": theta, "angle0": angle0, "angle_last": angle_last, "return_angle_last": return_angle_last,
            "B_last": B_last, "return_B_last": return_B_last}
    return _ssd_call(x, dt, lam, A, B, C, D, z, rope=rope, **kw)


def scan_step(u, delta, A, B, C, D=None, z=None, *, state, out_dtype=None, y=None, stream=None,
              dt_softplus: bool = False, dt_bias=None):
    """One selective-scan decode step (``ssm_scan_step``); ``state`` is updated
    in place.  Returns y.

    u, delta, z: (batch, dim); A: (dim, N) float32; B, C: (batch, G, N);
    D: (dim,) float32; state: (batch, dim, N) float32.
    """
    torch = _torch()
    in_code = _dtype_code(u.dtype)
    out_dt = u.dtype if out_dtype is None else out_dtype
    out_code = _dtype_code(out_dt)
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z)):
        if t is not None and t.dtype != u.dtype:
            raise TypeError(f"{name} must have dtype {u.dtype}")
    batch, dim = u.shape
    G, N = B.shape[1], B.shape[2]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("delta and z must have the shape of u")
    if B.shape != (batch, G, N) or C.shape != B.shape or A.shape != (dim, N):
        raise ValueError("B, C must be (batch, ngroups, dstate) and A (dim, dstate)")
    if state.dtype != torch.float32 or state.shape != (batch, dim, N):
        raise ValueError("state must be float32 (batch, dim, dstate)")
    with _alloc_on(stream):
        y = _out(y, (batch, dim), out_dt, u, "y")
    dims = StepDims(batch=batch, dim=dim, dstate=N, ngroups=G, in_dtype=in_code, out_dtype=out_code,
                    flags=0, reserved=0)
    _phase0(dims, dim, dt_softplus, dt_bias)
    _check(lib().ssm_scan_step(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(state), _ptr(y), ctypes.byref(dims), _stream(stream)))
    return y


def ssd_step(x, dt, A, B, C, D=None, z=None, *, state, out_dtype=None, y=None, stream=None,
             dt_softplus: bool = False, dt_bias=None):
    """One scalar-decay SSD decode step (``ssd_step``); ``state`` is updated in
    place.  Returns y.

    x, z: (batch, H, P); dt: (batch, H); A, D: (H,) float32; B, C: (batch, G, N);
    state: (batch, H, P, N) float32.
    """
    torch = _torch()
    in_code = _dtype_code(x.dtype)
    out_dt = x.dtype if out_dtype is None else out_dtype
    out_code = _dtype_code(out_dt)
    for name, t in (("dt", dt), ("B", B), ("C", C), ("z", z)):
        if t is not None and t.dtype != x.dtype:
            raise TypeError(f"{name} must have dtype {x.dtype}")
    batch, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    if dt.shape != (batch, H) or (z is not None and z.shape != x.shape):
        raise ValueError("dt must be (batch, H) and z shaped like x")
    if B.shape != (batch, G, N) or C.shape != B.shape or A.shape != (H,):
        raise ValueError("B, C must be (batch, ngroups, dstate) and A (nheads,)")
    if state.dtype != torch.float32 or state.shape != (batch, H, P, N):
        raise ValueError("state must be float32 (batch, nheads, headdim, dstate)")
    with _alloc_on(stream):
        y = _out(y, (batch, H, P), out_dt, x, "y")
    dims = SsdStepDims(batch=batch, nheads=H, headdim=P, dstate=N, ngroups=G, in_dtype=in_code,
                       out_dtype=out_code, flags=0, reserved=0)
    _phase0(dims, H, dt_softplus, dt_bias)
    _check(lib().ssd_step(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                          _ptr(state), _ptr(y), ctypes.byref(dims), _stream(stream)))
    return y


def ssd_trap_step(x, dt, lam, A, B, C, D=None, z=None, *, state, x_prev=None, B_prev=None, out_dtype=None,
                  y=None, stream=None, dt_softplus: bool = False, dt_bias=None, lam_sigmoid: bool = False):
    """One trapezoidal SSD decode step (``ssd_trap_step``); ``state`` is
    updated in place.  Returns y.

    x, z: (batch, H, P); dt, lam: (batch, H); A, D: (H,) float32; B, C:
    (batch, G, N); state: (batch, H, P, N) float32; x_prev (batch, H, P) and
    B_prev (batch, G, N): the previous token's x and B (None for the first
    token of a sequence).
    """
    torch = _torch()
    in_code = _dtype_code(x.dtype)
    out_dt = x.dtype if out_dtype is None else out_dtype
    out_code = _dtype_code(out_dt)
    for name, t in (("dt", dt), ("lam", lam), ("B", B), ("C", C), ("z", z), ("x_prev", x_prev),
                    ("B_prev", B_prev)):
        if t is not None and t.dtype != x.dtype:
            raise TypeError(f"{name} must have dtype {x.dtype}")
    batch, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    if dt.shape != (batch, H) or lam.shape != (batch, H) or (z is not None and z.shape != x.shape):
        raise ValueError("dt and lam must be (batch, H) and z shaped like x")
    if B.shape != (batch, G, N) or C.shape != B.shape or A.shape != (H,):
        raise ValueError("B, C must be (batch, ngroups, dstate) and A (nheads,)")
    if (x_prev is None) != (B_prev is None):
        raise ValueError("x_prev and B_prev are given together or not at all")
    if x_prev is not None and (x_prev.shape != x.shape or B_prev.shape != B.shape):
        raise ValueError("x_prev must be shaped like x and B_prev like B")
    if state.dtype != torch.float32 or state.shape != (batch, H, P, N):
        raise ValueError("state must be float32 (batch, nheads, headdim, dstate)")
    with _alloc_on(stream):
        y = _out(y, (batch, H, P), out_dt, x, "y")
    dims = SsdStepDims(batch=batch, nheads=H, headdim=P, dstate=N, ngroups=G, in_dtype=in_code,
                       out_dtype=out_code, flags=0, reserved=0)
    _phase0(dims, H, dt_softplus, dt_bias, lam_sigmoid)
    _check(lib().ssd_trap_step(_ptr(x), _ptr(dt), _ptr(lam), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(x_prev), _ptr(B_prev), _ptr(state), _ptr(y), ctypes.byref(dims),
                               _stream(stream)))
    return y


def rope_bc(dt, theta, B, C, *, angle0=None, out_dtype=None, B_rot=None, C_rot=None, angle_last=None,
            return_angle_last: bool = True, stream=None, dt_softplus: bool = False, dt_bias=None):
    """Rotary step on B and C (``ssm_rope_bc``). Returns ``(B_rot, C_rot,
    angle_last)`` (angle_last None when not asked for).

    dt: (batch, L, H); theta: (batch, L, TH, N / 2) with TH 1 or H;
    B, C: (batch, L, G, N), all of one dtype; angle0, angle_last:
    (batch, H, N / 2) float32 (angle_last may be angle0, updated in place);
    B_rot, C_rot: (batch, L, H, N) in out_dtype (default: the input dtype),
    ready for the SSD with ngroups = H.
    """
    torch = _torch()
    in_code = _dtype_code(B.dtype)
    out_dt = B.dtype if out_dtype is None else out_dtype
    out_code = _dtype_code(out_dt)
    for name, t in (("dt", dt), ("theta", theta), ("C", C)):
        if t.dtype != B.dtype:
            raise TypeError(f"{name} must have dtype {B.dtype}")
    batch, L, G, N = B.shape
    H = dt.shape[2]
    TH = theta.shape[2]
    if dt.shape != (batch, L, H) or C.shape != B.shape or N % 2 != 0:
        raise ValueError("dt must be (batch, L, H), C shaped like B, dstate even")
    if theta.shape != (batch, L, TH, N // 2):
        raise ValueError("theta must be (batch, L, 1 or H, dstate / 2)")
    if angle0 is not None and (angle0.dtype != torch.float32 or angle0.shape != (batch, H, N // 2)):
        raise ValueError("angle0 must be float32 (batch, nheads, dstate / 2)")
    with _alloc_on(stream):
        B_rot = _out(B_rot, (batch, L, H, N), out_dt, B, "B_rot")
        C_rot = _out(C_rot, (batch, L, H, N), out_dt, B, "C_rot")
        if angle_last is not None or return_angle_last:
            angle_last = _out(angle_last, (batch, H, N // 2), torch.float32, B, "angle_last")
    dims = RopeDims(batch=batch, seqlen=L, nheads=H, ngroups=G, dstate=N, theta_heads=TH, in_dtype=in_code,
                    out_dtype=out_code, flags=0, reserved=0)
    _phase0(dims, H, dt_softplus, dt_bias)
    _check(lib().ssm_rope_bc(_ptr(dt), _ptr(theta), _ptr(B), _ptr(C), _ptr(angle0), _ptr(B_rot), _ptr(C_rot),
                             _ptr(angle_last), ctypes.byref(dims), _stream(stream)))
    return B_rot, C_rot, angle_last


def rope_bc_bwd_workspace_size(dims: RopeDims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ssm_rope_bc_bwd_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def rope_bc_bwd(dt, theta, B, C, *, dB_rot, dC_rot, angle0=None, dangle_last=None, workspace=None,
                return_dangle0: bool = True, stream=None, dt_softplus: bool = False, dt_bias=None, out=None):
    """Backward of the rotary step (``ssm_rope_bc_bwd``): gradients of a loss
    with upstream dB_rot, dC_rot ((batch, L, H, N), float32 or bf16: the
    forward's B_rot dtype) and dangle_last ((batch, H, N / 2) float32,
    optional).  dt, theta, B, C, angle0 as given to ``rope_bc``.  Returns a
    dict of float32 tensors: ddt (batch, L, H), dtheta (like theta), dB, dC
    (like B, C) and dangle0 (batch, H, N / 2; None with return_dangle0
    False).  With dt_softplus, ddt is the gradient of the raw dt.  ``out``: an
    optional dict of preallocated output tensors under those names."""
    torch = _torch()
    in_code = _dtype_code(B.dtype)
    g_code = _dtype_code(dB_rot.dtype)
    for name, t in (("dt", dt), ("theta", theta), ("C", C)):
        if t.dtype != B.dtype:
            raise TypeError(f"{name} must have dtype {B.dtype}")
    if dC_rot.dtype != dB_rot.dtype:
        raise TypeError("dC_rot must have the dtype of dB_rot")
    batch, L, G, N = B.shape
    H = dt.shape[2]
    TH = theta.shape[2]
    if dt.shape != (batch, L, H) or C.shape != B.shape or N % 2 != 0:
        raise ValueError("dt must be (batch, L, H), C shaped like B, dstate even")
    if theta.shape != (batch, L, TH, N // 2):
        raise ValueError("theta must be (batch, L, 1 or H, dstate / 2)")
    if dB_rot.shape != (batch, L, H, N) or dC_rot.shape != dB_rot.shape:
        raise ValueError("dB_rot and dC_rot must be (batch, L, nheads, dstate)")
    for name, t in (("angle0", angle0), ("dangle_last", dangle_last)):
        if t is not None and (t.dtype != torch.float32 or t.shape != (batch, H, N // 2)):
            raise ValueError(f"{name} must be float32 (batch, nheads, dstate / 2)")
    dims = RopeDims(batch=batch, seqlen=L, nheads=H, ngroups=G, dstate=N, theta_heads=TH, in_dtype=in_code,
                    out_dtype=g_code, flags=0, reserved=0)
    _phase0(dims, H, dt_softplus, dt_bias)
    need = rope_bc_bwd_workspace_size(dims)
    f32 = torch.float32
    dev = B.device
    with _alloc_on(stream):
        if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        o = out or {}
        g = {"ddt": _out(o.get("ddt"), (batch, L, H), f32, B, "ddt"),
             "dtheta": _out(o.get("dtheta"), theta.shape, f32, B, "dtheta"),
             "dB": _out(o.get("dB"), B.shape, f32, B, "dB"),
             "dC": _out(o.get("dC"), C.shape, f32, B, "dC"),
             "dangle0": _out(o.get("dangle0"), (batch, H, N // 2), f32, B, "dangle0") if return_dangle0 else None}
    ws_bytes = 0 if (need == 0 or workspace is None) else workspace.numel() * workspace.element_size()
    _check(lib().ssm_rope_bc_bwd(_ptr(dt), _ptr(theta), _ptr(B), _ptr(C), _ptr(angle0), _ptr(dB_rot),
                                 _ptr(dC_rot), _ptr(dangle_last), _ptr(g["ddt"]), _ptr(g["dtheta"]),
                                 _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dangle0"]),
                                 _ptr(workspace) if need > 0 else None, ws_bytes, ctypes.byref(dims),
                                 _stream(stream)))
    return g
