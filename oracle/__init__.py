"""Python entry to the float64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  The wrappers only widen
the stored input values to float64 and marshal pointers; all arithmetic is in
``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11"]
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """ctypes binding of one build of ``oracle.c`` (the default build, or a
    variant that a test compiles from edited source)."""

    def __init__(self, libpath: str):
        lib = ctypes.CDLL(libpath)
        i64, dp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_scan_f64.argtypes = [i64] * 5 + [dp] * 10
        lib.oracle_scan_f64.restype = ctypes.c_int
        lib.oracle_ssd_f64.argtypes = [i64] * 6 + [dp] * 10
        lib.oracle_ssd_trap_f64.argtypes = [i64] * 6 + [dp] * 13
        lib.oracle_ssd_trap_f64.restype = ctypes.c_int
        lib.oracle_scan_bwd_f64.argtypes = [i64] * 5 + [dp] * 18
        lib.oracle_scan_bwd_f64.restype = ctypes.c_int
        lib.oracle_ssd_f64.restype = ctypes.c_int
        lib.oracle_ssd_bwd_f64.argtypes = [i64] * 6 + [dp] * 18
        lib.oracle_ssd_bwd_f64.restype = ctypes.c_int
        lib.oracle_ssd_trap_bwd_f64.argtypes = [i64] * 6 + [dp] * 24
        lib.oracle_ssd_trap_bwd_f64.restype = ctypes.c_int
        lib.oracle_softplus_f64.argtypes = [i64] * 3 + [dp] * 3
        lib.oracle_softplus_f64.restype = None
        lib.oracle_softplus_grad_f64.argtypes = [i64] * 3 + [dp] * 4
        lib.oracle_softplus_grad_f64.restype = None
        lib.oracle_sigmoid_f64.argtypes = [i64] + [dp] * 2
        lib.oracle_sigmoid_f64.restype = None
        lib.oracle_rope_bc_f64.argtypes = [i64] * 6 + [dp] * 8
        lib.oracle_rope_bc_f64.restype = ctypes.c_int
        lib.oracle_rope_bc_bwd_f64.argtypes = [i64] * 6 + [dp] * 13
        lib.oracle_rope_bc_bwd_f64.restype = ctypes.c_int
        self.lib = lib

    def rope_bc(self, dt, theta, B, C, angle0=None):
        """Rotary step on B and C in float64. Returns (B_rot, C_rot, angle_last).

        dt: (batch, L, H) (the step); theta: (batch, L, TH, N / 2) with TH 1 or H;
        B, C: (batch, L, G, N); angle0, angle_last: (batch, H, N / 2);
        B_rot, C_rot: (batch, L, H, N).
        """
        dt, theta, B, C, angle0 = map(f64, (dt, theta, B, C, angle0))
        batch, L, H = dt.shape
        G, N = B.shape[2], B.shape[3]
        TH = theta.shape[2]
        assert B.shape == (batch, L, G, N) and C.shape == B.shape
        assert theta.shape == (batch, L, TH, N // 2)
        assert angle0 is None or angle0.shape == (batch, H, N // 2)
        b_rot = np.zeros((batch, L, H, N))
        c_rot = np.zeros((batch, L, H, N))
        last = np.zeros((batch, H, N // 2))
        rc = self.lib.oracle_rope_bc_f64(batch, L, H, G, N, TH, _ptr(dt), _ptr(theta), _ptr(B), _ptr(C),
                                         _ptr(angle0), _ptr(b_rot), _ptr(c_rot), _ptr(last))
        if rc != 0:
            raise ValueError("oracle_rope_bc_f64 rejected the shapes")
        return b_rot, c_rot, last

    def rope_bc_bwd(self, dt, theta, B, C, angle0=None, dB_rot=None, dC_rot=None, dangle_last=None):
        """Gradients of ``rope_bc`` in float64 for upstream dB_rot, dC_rot
        (batch, L, H, N; None = zero) and dangle_last (batch, H, N / 2; None =
        zero).  Returns a dict: ddt (batch, L, H), dtheta (like theta), dB, dC
        (like B, C), dangle0 (batch, H, N / 2)."""
        dt, theta, B, C, angle0, dB_rot, dC_rot, dangle_last = map(
            f64, (dt, theta, B, C, angle0, dB_rot, dC_rot, dangle_last))
        batch, L, H = dt.shape
        G, N = B.shape[2], B.shape[3]
        TH = theta.shape[2]
        assert B.shape == (batch, L, G, N) and C.shape == B.shape
        assert theta.shape == (batch, L, TH, N // 2)
        zeros_rot = np.zeros((batch, L, H, N))
        dB_rot = zeros_rot if dB_rot is None else dB_rot
        dC_rot = zeros_rot if dC_rot is None else dC_rot
        assert dB_rot.shape == (batch, L, H, N) and dC_rot.shape == dB_rot.shape
        g = {"ddt": np.zeros((batch, L, H)), "dtheta": np.zeros(theta.shape), "dB": np.zeros(B.shape),
             "dC": np.zeros(C.shape), "dangle0": np.zeros((batch, H, N // 2))}
        rc = self.lib.oracle_rope_bc_bwd_f64(batch, L, H, G, N, TH, _ptr(dt), _ptr(theta), _ptr(B), _ptr(C),
                                             _ptr(angle0), _ptr(dB_rot), _ptr(dC_rot), _ptr(dangle_last),
                                             _ptr(g["ddt"]), _ptr(g["dtheta"]), _ptr(g["dB"]), _ptr(g["dC"]),
                                             _ptr(g["dangle0"]))
        if rc != 0:
            raise ValueError("oracle_rope_bc_bwd_f64 rejected the shapes")
        return g

    def softplus(self, raw, bias, inner):
        """Phase-0 step: softplus(raw + bias[(i / inner) % len(bias)]) elementwise
        over the flattened raw array (bias None: 0)."""
        raw, bias = f64(raw), f64(bias)
        out = np.empty_like(raw)
        nb = 1 if bias is None else bias.size
        self.lib.oracle_softplus_f64(raw.size, inner, nb, _ptr(raw), _ptr(bias), _ptr(out))
        return out

    def softplus_grad(self, raw, bias, inner, grad):
        """grad * sigmoid(raw + bias), the chain rule through ``softplus``."""
        raw, bias, grad = f64(raw), f64(bias), f64(grad)
        out = np.empty_like(raw)
        nb = 1 if bias is None else bias.size
        self.lib.oracle_softplus_grad_f64(raw.size, inner, nb, _ptr(raw), _ptr(bias), _ptr(grad), _ptr(out))
        return out

    def sigmoid(self, raw):
        """Phase-0 trapezoid weight: 1 / (1 + exp(-raw)) elementwise."""
        raw = f64(raw)
        out = np.empty_like(raw)
        self.lib.oracle_sigmoid_f64(raw.size, _ptr(raw), _ptr(out))
        return out

    def scan(self, u, delta, A, B, C, D=None, z=None, h0=None):
        """Selective scan in float64. Returns (y, h_last) as float64 arrays.

        u, delta, z: (batch, dim, L); B, C: (batch, G, N, L); A: (dim, N);
        D: (dim,); h0: (batch, dim, N).
        """
        u, delta, A, B, C, D, z, h0 = map(f64, (u, delta, A, B, C, D, z, h0))
        batch, dim, L = u.shape
        G, N = B.shape[1], B.shape[2]
        assert delta.shape == u.shape and A.shape == (dim, N) and C.shape == B.shape
        assert B.shape == (batch, G, N, L)
        assert z is None or z.shape == u.shape
        assert h0 is None or h0.shape == (batch, dim, N)
        y = np.zeros_like(u)
        h = np.zeros((batch, dim, N))
        rc = self.lib.oracle_scan_f64(batch, dim, N, L, G, _ptr(u), _ptr(delta), _ptr(A),
                                      _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                      _ptr(y), _ptr(h))
        if rc != 0:
            raise ValueError("oracle_scan_f64 rejected the shapes")
        return y, h

    def ssd_trap(self, x, dt, lam, A, B, C, D=None, z=None, h0=None, x_prev=None, B_prev=None):
        """Trapezoidal (three-term) SSD in float64. Returns (y, h_last).

        x, z: (batch, L, H, P); dt, lam: (batch, L, H); B, C: (batch, L, G, N);
        A, D: (H,); h0, h_last: (batch, H, P, N); x_prev (batch, H, P) and
        B_prev (batch, G, N): the token before the sequence (both or neither).
        """
        x, dt, lam, A, B, C, D, z, h0 = map(f64, (x, dt, lam, A, B, C, D, z, h0))
        x_prev, B_prev = f64(x_prev), f64(B_prev)
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        assert dt.shape == (batch, L, H) and lam.shape == dt.shape and A.shape == (H,)
        assert B.shape == (batch, L, G, N) and C.shape == B.shape
        assert h0 is None or h0.shape == (batch, H, P, N)
        assert (x_prev is None) == (B_prev is None)
        assert x_prev is None or (x_prev.shape == (batch, H, P) and B_prev.shape == (batch, G, N))
        y = np.zeros_like(x)
        h = np.zeros((batch, H, P, N))
        rc = self.lib.oracle_ssd_trap_f64(batch, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(lam), _ptr(A),
                                          _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(x_prev),
                                          _ptr(B_prev), _ptr(y), _ptr(h))
        if rc != 0:
            raise ValueError("oracle_ssd_trap_f64 rejected the shapes")
        return y, h

    def scan_bwd(self, u, delta, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None):
        """Gradients of the selective scan in float64 for upstream gradients dy
        (batch, dim, L) and dh_last (batch, dim, N; None = zero).  Returns a
        dict: du, ddelta, dA, dB, dC, and dD / dz / dh0 (dD, dz None when D, z
        are None)."""
        u, delta, A, B, C, D, z, h0, dy, dh_last = map(f64, (u, delta, A, B, C, D, z, h0, dy, dh_last))
        batch, dim, L = u.shape
        G, N = B.shape[1], B.shape[2]
        assert delta.shape == u.shape and A.shape == (dim, N) and C.shape == B.shape
        assert B.shape == (batch, G, N, L) and dy.shape == u.shape
        assert dh_last is None or dh_last.shape == (batch, dim, N)
        g = {"du": np.zeros_like(u), "ddelta": np.zeros_like(u), "dA": np.zeros((dim, N)),
             "dB": np.zeros_like(B), "dC": np.zeros_like(C),
             "dD": None if D is None else np.zeros(dim), "dz": None if z is None else np.zeros_like(u),
             "dh0": np.zeros((batch, dim, N))}
        rc = self.lib.oracle_scan_bwd_f64(batch, dim, N, L, G, _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                          _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_last),
                                          _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                                          _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]))
        if rc != 0:
            raise ValueError("oracle_scan_bwd_f64 rejected the shapes")
        return g

    def ssd_bwd(self, x, dt, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None):
        """Gradients of the scalar-decay SSD in float64 for upstream gradients
        dy (batch, L, H, P) and dh_last (batch, H, P, N; None = zero).  Returns a
        dict: dx, ddt, dA, dB, dC, dh0, and dD / dz (None when D / z are None)."""
        x, dt, A, B, C, D, z, h0, dy, dh_last = map(f64, (x, dt, A, B, C, D, z, h0, dy, dh_last))
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        assert dt.shape == (batch, L, H) and B.shape == (batch, L, G, N) and C.shape == B.shape
        assert A.shape == (H,) and dy.shape == x.shape
        assert h0 is None or h0.shape == (batch, H, P, N)
        assert dh_last is None or dh_last.shape == (batch, H, P, N)
        g = {"dx": np.zeros_like(x), "ddt": np.zeros_like(dt), "dA": np.zeros(H), "dB": np.zeros_like(B),
             "dC": np.zeros_like(C), "dD": None if D is None else np.zeros(H),
             "dz": None if z is None else np.zeros_like(x), "dh0": np.zeros((batch, H, P, N))}
        rc = self.lib.oracle_ssd_bwd_f64(batch, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                         _ptr(D), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(g["dx"]),
                                         _ptr(g["ddt"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                                         _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]))
        if rc != 0:
            raise ValueError("oracle_ssd_bwd_f64 rejected the shapes")
        return g

    def ssd_trap_bwd(self, x, dt, lam, A, B, C, D=None, z=None, h0=None, x_prev=None, B_prev=None, dy=None,
                     dh_last=None):
        """Gradients of the trapezoidal SSD in float64 for upstream gradients
        dy (batch, L, H, P) and dh_last (batch, H, P, N; None = zero).  Returns a
        dict: dx, ddt, dlam, dA, dB, dC, dh0, and dD / dz / dx_prev / dB_prev
        (None when D / z / the previous token are None)."""
        x, dt, lam, A, B, C, D, z, h0, dy, dh_last = map(f64, (x, dt, lam, A, B, C, D, z, h0, dy, dh_last))
        x_prev, B_prev = f64(x_prev), f64(B_prev)
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        assert dt.shape == (batch, L, H) and lam.shape == dt.shape and A.shape == (H,)
        assert B.shape == (batch, L, G, N) and C.shape == B.shape and dy.shape == x.shape
        assert h0 is None or h0.shape == (batch, H, P, N)
        assert dh_last is None or dh_last.shape == (batch, H, P, N)
        assert (x_prev is None) == (B_prev is None)
        g = {"dx": np.zeros_like(x), "ddt": np.zeros_like(dt), "dlam": np.zeros_like(dt), "dA": np.zeros(H),
             "dB": np.zeros_like(B), "dC": np.zeros_like(C), "dD": None if D is None else np.zeros(H),
             "dz": None if z is None else np.zeros_like(x), "dh0": np.zeros((batch, H, P, N)),
             "dx_prev": None if x_prev is None else np.zeros((batch, H, P)),
             "dB_prev": None if B_prev is None else np.zeros((batch, G, N))}
        rc = self.lib.oracle_ssd_trap_bwd_f64(batch, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(lam), _ptr(A), _ptr(B),
                                              _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(x_prev), _ptr(B_prev),
                                              _ptr(dy), _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddt"]),
                                              _ptr(g["dlam"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                                              _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]), _ptr(g["dx_prev"]),
                                              _ptr(g["dB_prev"]))
        if rc != 0:
            raise ValueError("oracle_ssd_trap_bwd_f64 rejected the shapes")
        return g

    def ssd(self, x, dt, A, B, C, D=None, z=None, h0=None):
        """Scalar-decay SSD recurrence in float64. Returns (y, h_last).

        x, z: (batch, L, H, P); dt: (batch, L, H); B, C: (batch, L, G, N);
        A, D: (H,); h0, h_last: (batch, H, P, N).
        """
        x, dt, A, B, C, D, z, h0 = map(f64, (x, dt, A, B, C, D, z, h0))
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        assert dt.shape == (batch, L, H) and B.shape == (batch, L, G, N)
        assert C.shape == B.shape and A.shape == (H,)
        assert h0 is None or h0.shape == (batch, H, P, N)
        y = np.zeros_like(x)
        h = np.zeros((batch, H, P, N))
        rc = self.lib.oracle_ssd_f64(batch, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A),
                                     _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                     _ptr(y), _ptr(h))
        if rc != 0:
            raise ValueError("oracle_ssd_f64 rejected the shapes")
        return y, h


def _load() -> Oracle:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = Oracle(_LIB)
    return _lib


def f64(a):
    """Widen a stored tensor/array (f32, bf16 or f64) to a contiguous float64 array."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (bf16 has no numpy dtype)
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data


def scan(u, delta, A, B, C, D=None, z=None, h0=None, dt_softplus=False, dt_bias=None):
    """Selective scan in float64 with the default build; see ``Oracle.scan``.
    dt_softplus: delta holds raw values and the step is softplus(delta +
    dt_bias[d]) (the Phase-0 map; dt_bias (dim,) or None)."""
    o = _load()
    if dt_softplus:
        delta = o.softplus(delta, dt_bias, f64(u).shape[2]).reshape(f64(u).shape)
    return o.scan(u, delta, A, B, C, D, z, h0)


def scan_bwd(u, delta, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None, dt_softplus=False,
             dt_bias=None):
    """Selective-scan gradients in float64 with the default build; see
    ``Oracle.scan_bwd``.  With dt_softplus the forward steps with
    softplus(delta + dt_bias) and ddelta is the gradient of the raw delta."""
    o = _load()
    if not dt_softplus:
        return o.scan_bwd(u, delta, A, B, C, D, z, h0, dy, dh_last)
    L = f64(u).shape[2]
    step = o.softplus(delta, dt_bias, L).reshape(f64(u).shape)
    g = o.scan_bwd(u, step, A, B, C, D, z, h0, dy, dh_last)
    g["ddelta"] = o.softplus_grad(delta, dt_bias, L, g["ddelta"]).reshape(step.shape)
    return g


def ssd_trap(x, dt, lam, A, B, C, D=None, z=None, h0=None, dt_softplus=False, dt_bias=None,
             lam_sigmoid=False, x_prev=None, B_prev=None):
    """Trapezoidal SSD in float64 with the default build; see ``Oracle.ssd_trap``.
    dt_softplus / lam_sigmoid: dt and lam hold raw values (Phase-0 maps).
    x_prev, B_prev: the token before the sequence (its previous-token term)."""
    o = _load()
    if dt_softplus:
        dt = o.softplus(dt, dt_bias, 1).reshape(f64(dt).shape)
    if lam_sigmoid:
        lam = o.sigmoid(lam).reshape(f64(lam).shape)
    return o.ssd_trap(x, dt, lam, A, B, C, D, z, h0, x_prev, B_prev)


def ssd_trap_step(x, dt, lam, A, B, C, D=None, z=None, state=None, x_prev=None, B_prev=None,
                  dt_softplus=False, dt_bias=None, lam_sigmoid=False):
    """One decode step of the trapezoidal SSD: ``ssd_trap`` with seqlen 1,
    h0 = state and the previous token's x_prev (batch, H, P) and B_prev
    (batch, G, N).  x, z: (batch, H, P); dt, lam: (batch, H); B, C:
    (batch, G, N); state: (batch, H, P, N).  Returns (y (batch, H, P), new state)."""
    row = lambda a: None if a is None else f64(a)[:, None]
    y, h = ssd_trap(row(x), row(dt), row(lam), A, row(B), row(C), D, row(z), state, dt_softplus, dt_bias,
                    lam_sigmoid, x_prev, B_prev)
    return y[:, 0], h


def ssd_bwd(x, dt, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None, dt_softplus=False, dt_bias=None):
    """Scalar-decay SSD gradients in float64 with the default build; see
    ``Oracle.ssd_bwd``.  With dt_softplus the forward steps with
    softplus(dt + dt_bias[h]) and ddt is the gradient of the raw dt."""
    o = _load()
    if not dt_softplus:
        return o.ssd_bwd(x, dt, A, B, C, D, z, h0, dy, dh_last)
    step = o.softplus(dt, dt_bias, 1).reshape(f64(dt).shape)
    g = o.ssd_bwd(x, step, A, B, C, D, z, h0, dy, dh_last)
    g["ddt"] = o.softplus_grad(dt, dt_bias, 1, g["ddt"]).reshape(step.shape)
    return g


def ssd_trap_bwd(x, dt, lam, A, B, C, D=None, z=None, h0=None, x_prev=None, B_prev=None, dy=None, dh_last=None,
                 dt_softplus=False, dt_bias=None, lam_sigmoid=False):
    """Trapezoidal SSD gradients in float64 with the default build; see
    ``Oracle.ssd_trap_bwd``.  With dt_softplus / lam_sigmoid the forward maps
    the raw dt and lam, and ddt / dlam are the gradients of the raw values
    (times sigmoid(dt + dt_bias[h]), and sigmoid'(lam) = s (1 - s))."""
    o = _load()
    step = o.softplus(dt, dt_bias, 1).reshape(f64(dt).shape) if dt_softplus else dt
    weight = o.sigmoid(lam).reshape(f64(lam).shape) if lam_sigmoid else lam
    g = o.ssd_trap_bwd(x, step, weight, A, B, C, D, z, h0, x_prev, B_prev, dy, dh_last)
    if dt_softplus:
        g["ddt"] = o.softplus_grad(dt, dt_bias, 1, g["ddt"]).reshape(step.shape)
    if lam_sigmoid:
        g["dlam"] = g["dlam"] * weight * (1.0 - weight)
    return g


def ssd(x, dt, A, B, C, D=None, z=None, h0=None, dt_softplus=False, dt_bias=None):
    """Scalar-decay SSD in float64 with the default build; see ``Oracle.ssd``.
    dt_softplus: dt holds raw values and the step is softplus(dt + dt_bias[h])."""
    o = _load()
    if dt_softplus:
        dt = o.softplus(dt, dt_bias, 1).reshape(f64(dt).shape)
    return o.ssd(x, dt, A, B, C, D, z, h0)


def scan_step(u, delta, A, B, C, D=None, z=None, state=None, dt_softplus=False, dt_bias=None):
    """One decode step of the selective scan: the recurrence at a single token
    from the cached ``state`` (zero when None), i.e. ``scan`` with seqlen 1 and
    h0 = state.  u, delta, z: (batch, dim); B, C: (batch, G, N);
    state: (batch, dim, N).  Returns (y (batch, dim), new state)."""
    col = lambda a: None if a is None else f64(a)[..., None]
    y, h = scan(col(u), col(delta), A, col(B), col(C), D, col(z), state, dt_softplus, dt_bias)
    return y[..., 0], h


def ssd_step(x, dt, A, B, C, D=None, z=None, state=None, dt_softplus=False, dt_bias=None):
    """One decode step of the scalar-decay SSD: ``ssd`` with seqlen 1 and
    h0 = state.  x, z: (batch, H, P); dt: (batch, H); B, C: (batch, G, N);
    state: (batch, H, P, N).  Returns (y (batch, H, P), new state)."""
    row = lambda a: None if a is None else f64(a)[:, None]
    y, h = ssd(row(x), row(dt), A, row(B), row(C), D, row(z), state, dt_softplus, dt_bias)
    return y[:, 0], h


def rope_bc(dt, theta, B, C, angle0=None, dt_softplus=False, dt_bias=None):
    """Rotary step on B and C in float64 with the default build; see
    ``Oracle.rope_bc``.  dt_softplus: dt holds raw values and the step is
    softplus(dt + dt_bias[h])."""
    o = _load()
    if dt_softplus:
        dt = o.softplus(dt, dt_bias, 1).reshape(f64(dt).shape)
    return o.rope_bc(dt, theta, B, C, angle0)


def rope_bc_bwd(dt, theta, B, C, angle0=None, dB_rot=None, dC_rot=None, dangle_last=None, dt_softplus=False,
                dt_bias=None):
    """Gradients of the rotary step in float64 with the default build; see
    ``Oracle.rope_bc_bwd``.  With dt_softplus the forward steps with
    softplus(dt + dt_bias[h]) and ddt is the gradient of the raw dt."""
    o = _load()
    if not dt_softplus:
        return o.rope_bc_bwd(dt, theta, B, C, angle0, dB_rot, dC_rot, dangle_last)
    step = o.softplus(dt, dt_bias, 1).reshape(f64(dt).shape)
    g = o.rope_bc_bwd(step, theta, B, C, angle0, dB_rot, dC_rot, dangle_last)
    g["ddt"] = o.softplus_grad(dt, dt_bias, 1, g["ddt"]).reshape(step.shape)
    return g
