"""fp64 CPU oracle of the selective scan (ctypes binding of ``oracle.c``).

TEST INFRASTRUCTURE ONLY: only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package. The HIP product path
never imports it and shares no code with it.

Every function takes the exact values handed to the GPU (float32 arrays that
hold fp32 or bf16-representable numbers), upcasts them to float64 and returns
a float64 result.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

ORD_FORWARD, ORD_REVERSE, ORD_COLUMN, ORD_COLUMN_REVERSE = 0, 1, 2, 3


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``oracle.c`` with gcc (IEEE double throughout, no fast-math)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", src, "-o", tmp,
                        "-lm", "-lpthread"], check=True)
        os.replace(tmp, out)
    return out


def load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    Lg = ctypes.c_long
    lib.oracle_scan_f64.argtypes = [I, I, I, Lg, Lg, Lg, I, P, P, P, P, P, P, I, P, P, P, I, P, I]
    lib.oracle_scan_f64.restype = I
    lib.oracle_scan_ex_f64.argtypes = [I, I, I, Lg, Lg, Lg, I, P, P, I, P, P, P, P, I, P, P, P, I,
                                       P, I]
    lib.oracle_scan_ex_f64.restype = I
    lib.oracle_vim_conv_f64.argtypes = [I, I, I, Lg, P, P, P, P, P, P, P, P, P, P, I, P, I]
    lib.oracle_vim_conv_f64.restype = I
    lib.oracle_vim_bidir_grad_f64.argtypes = [I, I, I, Lg] + [P] * 8 + [I] + [P] * 9 + [I]
    lib.oracle_vim_bidir_grad_f64.restype = I
    lib.oracle_linear_f64.argtypes = [I, I, I, Lg, P, P, P, P, P]
    lib.oracle_linear_f64.restype = I
    lib.oracle_dt_proj_f64.argtypes = [I, I, Lg, P, P, P]
    lib.oracle_dt_proj_f64.restype = I
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan(u, delta, z, B, C, A, Dskip, dt_bias, *, orders: Sequence[int],
         bc_per_direction: bool, H: int = 0, W: int = 0, delta_softplus: bool = True,
         nthreads: Optional[int] = None, lib=None, u_per_direction: bool = False,
         delta_per_direction: bool = False, zoh: bool = False) -> np.ndarray:
    """Generic scan: len(orders) directions, merged by sum, optional gate.

    u, delta, z: [batch, dim, L] (u, delta: [ndir, batch, dim, L] when
    u_per_direction, delta_per_direction); B, C: [batch, dstate, L] (shared, token order) or
    [batch, ndir, dstate, L] (per direction, scan order);
    A: [ndir, dim, dstate]; Dskip, dt_bias: [ndir, dim] or None.
    """
    lib = lib or load()
    u, delta, z, B, C, A = map(_f64, (u, delta, z, B, C, A))
    Dskip, dt_bias = _f64(Dskip), _f64(dt_bias)
    batch, dim, L = delta.shape[-3:]
    ndir = len(orders)
    assert u.shape == ((ndir,) if u_per_direction else ()) + (batch, dim, L)
    assert delta.shape == ((ndir,) if delta_per_direction else ()) + (batch, dim, L)
    dstate = A.shape[-1]
    assert z is None or z.shape == (batch, dim, L)
    assert A.shape == (ndir, dim, dstate)
    if bc_per_direction:
        assert B.shape == (batch, ndir, dstate, L) and C.shape == B.shape
    else:
        assert B.shape == (batch, dstate, L) and C.shape == B.shape
    for p in (Dskip, dt_bias):
        assert p is None or p.shape == (ndir, dim)
    order = np.ascontiguousarray(orders, dtype=np.intc)
    y = np.empty((batch, dim, L), np.float64)
    rc = lib.oracle_scan_ex_f64(batch, dim, dstate, L, H, W, ndir, _ptr(order), _ptr(u),
                                int(bool(u_per_direction)) | (2 if delta_per_direction else 0),
                                _ptr(delta), _ptr(z), _ptr(B),
                                _ptr(C), int(bc_per_direction), _ptr(A), _ptr(Dskip),
                                _ptr(dt_bias), int(bool(delta_softplus)) | (2 if zoh else 0),
                                _ptr(y), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_scan_ex_f64 failed with status %d" % rc)
    return y


def vim_dirs(u, delta, z, B, C, A, Dskip, dt_bias, delta_softplus=True, nthreads=None,
             zoh=False):
    """Vim with per-direction inputs (the guide's block code gives each branch
    its own conv and SimpleSelectiveSSM, hence its own u, delta, B, C):
    u, delta [2, batch, dim, L] and B, C [batch, 2, dstate, L], all in token
    order; z [batch, dim, L] (shared gate) or None. The backward direction
    visits token L-1-t at step t, so its B, C are passed to the scan in that
    order (a flip)."""
    B, C = _f64(B), _f64(C)
    Bs, Cs = B.copy(), C.copy()
    Bs[:, 1] = B[:, 1, :, ::-1]
    Cs[:, 1] = C[:, 1, :, ::-1]
    return scan(u, delta, z, Bs, Cs, A, Dskip, dt_bias, orders=(ORD_FORWARD, ORD_REVERSE),
                bc_per_direction=True, delta_softplus=delta_softplus, nthreads=nthreads,
                u_per_direction=True, delta_per_direction=True, zoh=zoh)


def vim_bidir(u, delta, z, B, C, A, Dskip, dt_bias, delta_softplus=True, nthreads=None,
              zoh=False):
    """Vim: forward + backward over shared u, delta, z, B, C."""
    return scan(u, delta, z, B, C, A, Dskip, dt_bias, orders=(ORD_FORWARD, ORD_REVERSE),
                bc_per_direction=False, delta_softplus=delta_softplus, nthreads=nthreads,
                zoh=zoh)


def vim_conv(x, conv_w, conv_b, delta, z, B, C, A, Dskip, dt_bias, delta_softplus=True,
             nthreads=None, lib=None, zoh=False):
    """Vim with its conv front end: u_f = silu(conv_f(x)), u_b the flipped
    branch's silu(conv_b(flip x)). x: [batch, dim, L]; conv_w: [2, dim, 3];
    conv_b: [2, dim] or None; the rest as for vim_bidir."""
    lib = lib or load()
    x, conv_w, conv_b, delta, z, B, C, A = map(_f64, (x, conv_w, conv_b, delta, z, B, C, A))
    Dskip, dt_bias = _f64(Dskip), _f64(dt_bias)
    batch, dim, L = x.shape
    dstate = A.shape[-1]
    assert conv_w.shape == (2, dim, 3) and (conv_b is None or conv_b.shape == (2, dim))
    assert delta.shape == x.shape and (z is None or z.shape == x.shape)
    assert A.shape == (2, dim, dstate) and B.shape == (batch, dstate, L) and C.shape == B.shape
    y = np.empty((batch, dim, L), np.float64)
    rc = lib.oracle_vim_conv_f64(batch, dim, dstate, L, _ptr(x), _ptr(conv_w), _ptr(conv_b),
                                 _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
                                 _ptr(dt_bias), int(bool(delta_softplus)) | (2 if zoh else 0),
                                 _ptr(y),
                                 nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_vim_conv_f64 failed with status %d" % rc)
    return y


GRAD_NAMES = ("du", "ddelta", "dz", "dB", "dC", "dA", "dD", "ddt_bias")


def vim_bidir_grad(u, delta, z, B, C, A, Dskip, dt_bias, g, delta_softplus=True, nthreads=None,
                   lib=None):
    """Gradient of vim_bidir's output against an upstream gradient g (same
    shape as y). Returns a dict: du, ddelta, dz [batch, dim, L]; dB, dC
    [batch, dstate, L]; dA [2, dim, dstate]; dD, ddt_bias [2, dim] (dz is 0
    without a gate)."""
    lib = lib or load()
    u, delta, z, B, C, A, g = map(_f64, (u, delta, z, B, C, A, g))
    Dskip, dt_bias = _f64(Dskip), _f64(dt_bias)
    batch, dim, L = u.shape
    dstate = A.shape[-1]
    assert delta.shape == u.shape and g.shape == u.shape and (z is None or z.shape == u.shape)
    assert A.shape == (2, dim, dstate) and B.shape == (batch, dstate, L) and C.shape == B.shape
    out = {k: np.empty(u.shape) for k in ("du", "ddelta", "dz")}
    out.update(dB=np.empty(B.shape), dC=np.empty(B.shape), dA=np.empty(A.shape),
               dD=np.empty((2, dim)), ddt_bias=np.empty((2, dim)))
    rc = lib.oracle_vim_bidir_grad_f64(batch, dim, dstate, L, _ptr(u), _ptr(delta), _ptr(z),
                                       _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip), _ptr(dt_bias),
                                       int(bool(delta_softplus)), _ptr(g),
                                       *[_ptr(out[k]) for k in GRAD_NAMES],
                                       nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_vim_bidir_grad_f64 failed with status %d" % rc)
    return out


def cross4(u, delta, z, B, C, A, Dskip, dt_bias, H, W, delta_softplus=True, nthreads=None,
           zoh=False):
    """VMamba cross-scan: row-major, reversed, column-major, reversed."""
    return scan(u, delta, z, B, C, A, Dskip, dt_bias,
                orders=(ORD_FORWARD, ORD_REVERSE, ORD_COLUMN, ORD_COLUMN_REVERSE),
                bc_per_direction=True, H=H, W=W, delta_softplus=delta_softplus, zoh=zoh,
                nthreads=nthreads)


def s6_1d(u, delta, z, B, C, A, Dskip, dt_bias, reverse=False, delta_softplus=True,
          nthreads=None, zoh=False):
    """A single direction. A: [dim, dstate]; Dskip, dt_bias: [dim] or None."""
    A = np.asarray(A)[None]
    Dskip = None if Dskip is None else np.asarray(Dskip)[None]
    dt_bias = None if dt_bias is None else np.asarray(dt_bias)[None]
    return scan(u, delta, z, B, C, A, Dskip, dt_bias,
                orders=(ORD_REVERSE if reverse else ORD_FORWARD,), bc_per_direction=False,
                delta_softplus=delta_softplus, nthreads=nthreads, zoh=zoh)


def run_inputs(inp, nthreads=None, zoh=False) -> np.ndarray:
    """The oracle on a ``workloads.Inputs`` bundle (the workload decides the kind)."""
    wl = inp.wl
    if wl.kind == "vim":
        return vim_bidir(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D, inp.dt_bias,
                         nthreads=nthreads, zoh=zoh)
    return cross4(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D, inp.dt_bias,
                  wl.H, wl.W, nthreads=nthreads, zoh=zoh)


# ---- the linear maps around the scan (x_proj, dt_proj, out_proj)
def linear(W, x, bias=None, residual=None, lib=None):
    """nn.Linear in the channel-major layout: out[b, m, t] = sum_k W[m, k]
    x[b, k, t] + bias[m] (+ residual[b, m, t]). W: [M, K]; x: [batch, K, L]."""
    lib = lib or load()
    W, x, bias, residual = map(_f64, (W, x, bias, residual))
    batch, K, L = x.shape
    M = W.shape[0]
    assert W.shape == (M, K) and (bias is None or bias.shape == (M,))
    assert residual is None or residual.shape == (batch, M, L)
    out = np.empty((batch, M, L), np.float64)
    rc = lib.oracle_linear_f64(batch, M, K, L, _ptr(W), _ptr(x), _ptr(bias), _ptr(residual),
                               _ptr(out))
    if rc != 0:
        raise ValueError("oracle_linear_f64 failed with status %d" % rc)
    return out


def x_proj(W, u, dstate, lib=None):
    """SimpleSelectiveSSM.x_proj on u [batch, dim, L] with W [2 dstate + 1, dim]:
    rows 0..N-1 of the projection are B, rows N..2N-1 are C, row 2N is dt
    (the code's proj[..., :N], proj[..., N:2N], proj[..., 2N:])."""
    p = linear(W, u, lib=lib)
    return p[:, :dstate], p[:, dstate:2 * dstate], p[:, 2 * dstate]


def dt_proj(dt, w, lib=None):
    """dt_proj without its bias (the scan's dt_bias adds it before the
    softplus): delta_raw[b, d, t] = w[d] dt[b, t]. dt: [batch, L]; w: [dim]."""
    lib = lib or load()
    dt, w = _f64(dt), _f64(w)
    batch, L = dt.shape
    dim = w.shape[0]
    out = np.empty((batch, dim, L), np.float64)
    rc = lib.oracle_dt_proj_f64(batch, dim, L, _ptr(dt), _ptr(w), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dt_proj_f64 failed with status %d" % rc)
    return out
