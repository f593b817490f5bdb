"""Torch-facing binding of the C ABI (same names as include/vimscan.h).

Torch provides device memory and the stream; the functions below only check
that tensors have the layouts the ABI expects and pass their pointers on.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _native as nat

_DTYPES = {torch.float32: nat.VS_F32, torch.bfloat16: nat.VS_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _flags(delta_softplus, zoh):
    """The flags word of the scan entry points: VS_FLAG_SOFTPLUS (1) and
    VS_FLAG_ZOH (2, the exact zero-order hold B_bar = (exp(delta A) - 1)/A B)."""
    return (1 if delta_softplus else 0) | (2 if zoh else 0)


def _act(name, t, shape, dtype, device):
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _param(name, t, shape, device, optional=True):
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    _act(name, t, shape, torch.float32, device)


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def workspace_bytes(op: int, batch: int, dim: int, seqlen: int, dtype: torch.dtype) -> int:
    return int(nat.lib.vs_workspace_bytes(op, batch, dim, seqlen, _DTYPES[dtype]))


def _workspace(op, batch, dim, seqlen, dtype, device, workspace):
    need = workspace_bytes(op, batch, dim, seqlen, dtype)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
        raise ValueError("workspace needs %d contiguous bytes" % need)
    return workspace, workspace.numel() * workspace.element_size()


def vim_scan_bidir(u, delta, z, B, C, A, Dskip=None, dt_bias=None, delta_softplus=True,
                   zoh=False, out=None, workspace=None):
    """Vim forward + backward selective scan, merged and gated.

    u, delta, z: [batch, dim, L] (fp32 or bf16; z may be None);
    B, C: [batch, dstate, L]; A: [2, dim, dstate] fp32; Dskip, dt_bias:
    [2, dim] fp32 or None. Returns y [batch, dim, L] in the input dtype.
    """
    batch, dim, L = u.shape
    dstate = A.shape[-1]
    dt, dev = u.dtype, u.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        if t is not None:
            _act(name, t, (batch, dim, L), dt, dev)
    _act("B", B, (batch, dstate, L), dt, dev)
    _act("C", C, (batch, dstate, L), dt, dev)
    _param("A", A, (2, dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (2, dim), dev)
    _param("dt_bias", dt_bias, (2, dim), dev)
    y = torch.empty_like(u) if out is None else out
    _act("out", y, (batch, dim, L), dt, dev)
    ws, ws_bytes = _workspace(nat.VS_OP_VIM_BIDIR, batch, dim, L, dt, dev, workspace)
    rc = nat.lib.vim_scan_bidir(batch, dim, dstate, L, _DTYPES[dt], _ptr(u), _ptr(delta), _ptr(z),
                                _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip), _ptr(dt_bias),
                                _flags(delta_softplus, zoh), _ptr(y), _ptr(ws), ws_bytes,
                                _stream(dev))
    nat.check("vim_scan_bidir", rc)
    return y


def vim_scan_bidir_chunked(u, delta, z, B, C, A, Dskip=None, dt_bias=None, chunks=0,
                           delta_softplus=True, out=None, workspace=None):
    """vim_scan_bidir with the sequence cut into `chunks` parallel pieces
    joined by the associative carry combine (0: the library's choice)."""
    batch, dim, L = u.shape
    dstate = A.shape[-1]
    dt, dev = u.dtype, u.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        if t is not None:
            _act(name, t, (batch, dim, L), dt, dev)
    _act("B", B, (batch, dstate, L), dt, dev)
    _act("C", C, (batch, dstate, L), dt, dev)
    _param("A", A, (2, dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (2, dim), dev)
    _param("dt_bias", dt_bias, (2, dim), dev)
    y = torch.empty_like(u) if out is None else out
    _act("out", y, (batch, dim, L), dt, dev)
    ws, ws_bytes = _workspace(nat.VS_OP_VIM_BIDIR, batch, dim, L, dt, dev, workspace)
    rc = nat.lib.vim_scan_bidir_chunked(batch, dim, dstate, L, _DTYPES[dt], _ptr(u), _ptr(delta),
                                        _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
                                        _ptr(dt_bias), _flags(delta_softplus, False), int(chunks),
                                        _ptr(y), _ptr(ws), ws_bytes, _stream(dev))
    nat.check("vim_scan_bidir_chunked", rc)
    return y


def vim_scan_bidir_noalloc(u, delta, z, B, C, A, Dskip=None, dt_bias=None, delta_softplus=True,
                           zoh=False, out=None):
    """vim_scan_bidir without a workspace: the merge buffer is the library's
    own static device array, so the call allocates nothing when `out` is
    given (bf16: batch*dim*L up to VS_NOALLOC_MAX_ELEMS). Calls that overlap
    on one GPU share that buffer and must be serialised."""
    batch, dim, L = u.shape
    dstate = A.shape[-1]
    dt, dev = u.dtype, u.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        if t is not None:
            _act(name, t, (batch, dim, L), dt, dev)
    _act("B", B, (batch, dstate, L), dt, dev)
    _act("C", C, (batch, dstate, L), dt, dev)
    _param("A", A, (2, dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (2, dim), dev)
    _param("dt_bias", dt_bias, (2, dim), dev)
    y = torch.empty_like(u) if out is None else out
    _act("out", y, (batch, dim, L), dt, dev)
    rc = nat.lib.vim_scan_bidir_noalloc(batch, dim, dstate, L, _DTYPES[dt], _ptr(u), _ptr(delta),
                                        _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
                                        _ptr(dt_bias), _flags(delta_softplus, zoh), _ptr(y),
                                        _stream(dev))
    nat.check("vim_scan_bidir_noalloc", rc)
    return y


def vim_scan_bidir_dirs(u, delta, z, B, C, A, Dskip=None, dt_bias=None, delta_softplus=True,
                        zoh=False, out=None, workspace=None):
    """vim_scan_bidir with per-direction inputs: u, delta [2, batch, dim, L]
    and B, C [batch, 2, dstate, L], token order (copy 0 forward, copy 1
    backward); z [batch, dim, L] or None. Returns y [batch, dim, L]."""
    _, batch, dim, L = u.shape
    dstate = A.shape[-1]
    dt, dev = u.dtype, u.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    _act("u", u, (2, batch, dim, L), dt, dev)
    _act("delta", delta, (2, batch, dim, L), dt, dev)
    if z is not None:
        _act("z", z, (batch, dim, L), dt, dev)
    _act("B", B, (batch, 2, dstate, L), dt, dev)
    _act("C", C, (batch, 2, dstate, L), dt, dev)
    _param("A", A, (2, dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (2, dim), dev)
    _param("dt_bias", dt_bias, (2, dim), dev)
    y = torch.empty(batch, dim, L, dtype=dt, device=dev) if out is None else out
    _act("out", y, (batch, dim, L), dt, dev)
    ws, ws_bytes = _workspace(nat.VS_OP_VIM_BIDIR, batch, dim, L, dt, dev, workspace)
    rc = nat.lib.vim_scan_bidir_dirs(batch, dim, dstate, L, _DTYPES[dt], _ptr(u), _ptr(delta),
                                     _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
                                     _ptr(dt_bias), _flags(delta_softplus, zoh), _ptr(y), _ptr(ws),
                                     ws_bytes, _stream(dev))
    nat.check("vim_scan_bidir_dirs", rc)
    return y


def vim_scan_bidir_conv(x, conv_w, conv_b, delta, z, B, C, A, Dskip=None, dt_bias=None,
                        delta_softplus=True, zoh=False, out=None, workspace=None):
    """vim_scan_bidir with the Vim block's conv front end fused in: each
    branch scans u_k = silu(conv_k(x)) (depthwise kernel 3, padding 1; the
    backward branch on the flipped sequence).

    x: [batch, dim, L]; conv_w: [2, dim, 3] fp32; conv_b: [2, dim] fp32 or
    None; the rest as for vim_scan_bidir.
    """
    batch, dim, L = x.shape
    dstate = A.shape[-1]
    dt, dev = x.dtype, x.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    for name, t in (("x", x), ("delta", delta), ("z", z)):
        if t is not None:
            _act(name, t, (batch, dim, L), dt, dev)
    _act("B", B, (batch, dstate, L), dt, dev)
    _act("C", C, (batch, dstate, L), dt, dev)
    _param("conv_w", conv_w, (2, dim, 3), dev, optional=False)
    _param("conv_b", conv_b, (2, dim), dev)
    _param("A", A, (2, dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (2, dim), dev)
    _param("dt_bias", dt_bias, (2, dim), dev)
    y = torch.empty_like(x) if out is None else out
    _act("out", y, (batch, dim, L), dt, dev)
    ws, ws_bytes = _workspace(nat.VS_OP_VIM_BIDIR, batch, dim, L, dt, dev, workspace)
    rc = nat.lib.vim_scan_bidir_conv(batch, dim, dstate, L, _DTYPES[dt], _ptr(x), _ptr(conv_w),
                                     _ptr(conv_b), _ptr(delta), _ptr(z), _ptr(B), _ptr(C),
                                     _ptr(A), _ptr(Dskip), _ptr(dt_bias),
                                     _flags(delta_softplus, zoh), _ptr(y), _ptr(ws), ws_bytes,
                                     _stream(dev))
    nat.check("vim_scan_bidir_conv", rc)
    return y


def vim_scan_bidir_grad(u, delta, z, B, C, A, Dskip, dt_bias, dy, delta_softplus=True,
                        workspace=None):
    """Gradient of vim_scan_bidir for an upstream gradient dy (same shape as
    y). Returns a dict: du, ddelta, dz (None without z) in the input dtype,
    [batch, dim, L]; dB, dC fp32 [batch, dstate, L]; dA fp32 [2, dim,
    dstate]; dD, ddt_bias fp32 [2, dim]."""
    batch, dim, L = u.shape
    dstate = A.shape[-1]
    dt, dev = u.dtype, u.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    for name, t in (("u", u), ("delta", delta), ("z", z), ("dy", dy)):
        if t is not None:
            _act(name, t, (batch, dim, L), dt, dev)
    _act("B", B, (batch, dstate, L), dt, dev)
    _act("C", C, (batch, dstate, L), dt, dev)
    _param("A", A, (2, dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (2, dim), dev)
    _param("dt_bias", dt_bias, (2, dim), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u),
               dz=None if z is None else torch.empty_like(u),
               dB=torch.empty(batch, dstate, L, **f32), dC=torch.empty(batch, dstate, L, **f32),
               dA=torch.empty(2, dim, dstate, **f32), dD=torch.empty(2, dim, **f32),
               ddt_bias=torch.empty(2, dim, **f32))
    ws, ws_bytes = _workspace(nat.VS_OP_VIM_GRAD, batch, dim, L, dt, dev, workspace)
    rc = nat.lib.vim_scan_bidir_grad(batch, dim, dstate, L, _DTYPES[dt], _ptr(u), _ptr(delta),
                                     _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
                                     _ptr(dt_bias), int(bool(delta_softplus)), _ptr(dy),
                                     _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dz"]),
                                     _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dA"]),
                                     _ptr(out["dD"]), _ptr(out["ddt_bias"]), _ptr(ws), ws_bytes,
                                     _stream(dev))
    nat.check("vim_scan_bidir_grad", rc)
    return out


def vim_scan_bidir_fwd_saved(u, delta, z, B, C, A, Dskip=None, dt_bias=None, delta_softplus=True,
                             out=None, saved=None):
    """vim_scan_bidir (delta B form) that also fills the saved-state buffer a
    later vim_scan_bidir_grad_saved call on the same inputs reads instead of
    re-running the forward pass. Returns (y, saved); saved is an opaque
    uint8 tensor of vs_workspace_bytes(VS_OP_VIM_SAVED) bytes."""
    batch, dim, L = u.shape
    dstate = A.shape[-1]
    dt, dev = u.dtype, u.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        if t is not None:
            _act(name, t, (batch, dim, L), dt, dev)
    _act("B", B, (batch, dstate, L), dt, dev)
    _act("C", C, (batch, dstate, L), dt, dev)
    _param("A", A, (2, dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (2, dim), dev)
    _param("dt_bias", dt_bias, (2, dim), dev)
    y = torch.empty_like(u) if out is None else out
    _act("out", y, (batch, dim, L), dt, dev)
    sv, sv_bytes = _workspace(nat.VS_OP_VIM_SAVED, batch, dim, L, dt, dev, saved)
    rc = nat.lib.vim_scan_bidir_fwd_saved(batch, dim, dstate, L, _DTYPES[dt], _ptr(u), _ptr(delta),
                                          _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
                                          _ptr(dt_bias), int(bool(delta_softplus)), _ptr(y), _ptr(sv),
                                          sv_bytes, _stream(dev))
    nat.check("vim_scan_bidir_fwd_saved", rc)
    return y, sv


def vim_scan_bidir_grad_saved(u, delta, z, B, C, A, Dskip, dt_bias, saved, dy, delta_softplus=True,
                              workspace=None):
    """vim_scan_bidir_grad with the forward pass read from `saved`, the buffer
    of a vim_scan_bidir_fwd_saved call on the same inputs. Returns the same
    dict as vim_scan_bidir_grad."""
    batch, dim, L = u.shape
    dstate = A.shape[-1]
    dt, dev = u.dtype, u.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    for name, t in (("u", u), ("delta", delta), ("z", z), ("dy", dy)):
        if t is not None:
            _act(name, t, (batch, dim, L), dt, dev)
    _act("B", B, (batch, dstate, L), dt, dev)
    _act("C", C, (batch, dstate, L), dt, dev)
    _param("A", A, (2, dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (2, dim), dev)
    _param("dt_bias", dt_bias, (2, dim), dev)
    need = workspace_bytes(nat.VS_OP_VIM_SAVED, batch, dim, L, dt)
    if (saved is None or saved.device != dev or not saved.is_contiguous()
            or saved.numel() * saved.element_size() < need):
        raise ValueError("saved must be the contiguous %d-byte buffer of vim_scan_bidir_fwd_saved" % need)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u),
               dz=None if z is None else torch.empty_like(u),
               dB=torch.empty(batch, dstate, L, **f32), dC=torch.empty(batch, dstate, L, **f32),
               dA=torch.empty(2, dim, dstate, **f32), dD=torch.empty(2, dim, **f32),
               ddt_bias=torch.empty(2, dim, **f32))
    ws, ws_bytes = _workspace(nat.VS_OP_VIM_GRAD_SAVED, batch, dim, L, dt, dev, workspace)
    rc = nat.lib.vim_scan_bidir_grad_saved(batch, dim, dstate, L, _DTYPES[dt], _ptr(u), _ptr(delta),
                                           _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
                                           _ptr(dt_bias), int(bool(delta_softplus)), _ptr(saved),
                                           saved.numel() * saved.element_size(), _ptr(dy),
                                           _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dz"]),
                                           _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dA"]),
                                           _ptr(out["dD"]), _ptr(out["ddt_bias"]), _ptr(ws), ws_bytes,
                                           _stream(dev))
    nat.check("vim_scan_bidir_grad_saved", rc)
    return out


def vmamba_cross_scan4(u, delta, z, B, C, A, H, W, Dskip=None, dt_bias=None,
                       delta_softplus=True, zoh=False, out=None, workspace=None):
    """VMamba four-direction cross-scan of an H x W grid.

    u, delta, z: [batch, dim, H*W] (row-major grid; z may be None);
    B, C: [batch, 4, dstate, H*W] in each direction's scan order;
    A: [4, dim, dstate]; Dskip, dt_bias: [4, dim] or None.
    """
    batch, dim, L = u.shape
    if H * W != L:
        raise ValueError("H*W must equal the token count")
    dstate = A.shape[-1]
    dt, dev = u.dtype, u.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        if t is not None:
            _act(name, t, (batch, dim, L), dt, dev)
    _act("B", B, (batch, 4, dstate, L), dt, dev)
    _act("C", C, (batch, 4, dstate, L), dt, dev)
    _param("A", A, (4, dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (4, dim), dev)
    _param("dt_bias", dt_bias, (4, dim), dev)
    y = torch.empty_like(u) if out is None else out
    _act("out", y, (batch, dim, L), dt, dev)
    ws, ws_bytes = _workspace(nat.VS_OP_CROSS4, batch, dim, L, dt, dev, workspace)
    rc = nat.lib.vmamba_cross_scan4(batch, dim, dstate, H, W, _DTYPES[dt], _ptr(u), _ptr(delta),
                                    _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
                                    _ptr(dt_bias), _flags(delta_softplus, zoh), _ptr(y), _ptr(ws),
                                    ws_bytes, _stream(dev))
    nat.check("vmamba_cross_scan4", rc)
    return y


def s6_scan_1d(u, delta, z, B, C, A, Dskip=None, dt_bias=None, reverse=False,
               delta_softplus=True, zoh=False, out=None):
    """One direction of the scan. A: [dim, dstate]; Dskip, dt_bias: [dim]."""
    batch, dim, L = u.shape
    dstate = A.shape[-1]
    dt, dev = u.dtype, u.device
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        if t is not None:
            _act(name, t, (batch, dim, L), dt, dev)
    _act("B", B, (batch, dstate, L), dt, dev)
    _act("C", C, (batch, dstate, L), dt, dev)
    _param("A", A, (dim, dstate), dev, optional=False)
    _param("Dskip", Dskip, (dim,), dev)
    _param("dt_bias", dt_bias, (dim,), dev)
    y = torch.empty_like(u) if out is None else out
    _act("out", y, (batch, dim, L), dt, dev)
    rc = nat.lib.s6_scan_1d(batch, dim, dstate, L, _DTYPES[dt], int(bool(reverse)), _ptr(u),
                            _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
                            _ptr(dt_bias), _flags(delta_softplus, zoh), _ptr(y), _stream(dev))
    nat.check("s6_scan_1d", rc)
    return y


# ---- the linear maps around the scan (bf16, matrix cores)
def _bf16_act(name, t, shape, dev):
    _act(name, t, shape, torch.bfloat16, dev)


def vim_x_proj(u, W, dstate):
    """SimpleSelectiveSSM.x_proj: u [batch, dim, L] bf16, W [2 dstate + 1, dim]
    bf16 -> (B [batch, dstate, L] bf16, C [batch, dstate, L] bf16,
    dt [batch, L] fp32)."""
    batch, dim, L = u.shape
    dev = u.device
    _bf16_act("u", u, (batch, dim, L), dev)
    _bf16_act("W", W, (2 * dstate + 1, dim), dev)
    B = torch.empty(batch, dstate, L, dtype=torch.bfloat16, device=dev)
    C = torch.empty_like(B)
    dt = torch.empty(batch, L, dtype=torch.float32, device=dev)
    rc = nat.lib.vim_x_proj(batch, dim, dstate, L, nat.VS_BF16, _ptr(u), _ptr(W), _ptr(B), _ptr(C),
                            _ptr(dt), _stream(dev))
    nat.check("vim_x_proj", rc)
    return B, C, dt


def vim_dt_proj(dt, w):
    """dt_proj without its bias (the scan's dt_bias): dt [batch, L] fp32,
    w [dim] fp32 -> delta_raw [batch, dim, L] bf16."""
    batch, L = dt.shape
    dim = w.shape[0]
    dev = dt.device
    _act("dt", dt, (batch, L), torch.float32, dev)
    _act("w", w, (dim,), torch.float32, dev)
    delta = torch.empty(batch, dim, L, dtype=torch.bfloat16, device=dev)
    rc = nat.lib.vim_dt_proj(batch, dim, L, nat.VS_BF16, _ptr(dt), _ptr(w), _ptr(delta),
                             _stream(dev))
    nat.check("vim_dt_proj", rc)
    return delta


def vim_out_proj(y, W, bias=None, residual=None, out=None):
    """out = W y + bias + residual: y [batch, dim_in, L] bf16, W [dim_out,
    dim_in] bf16, bias [dim_out] fp32 or None, residual [batch, dim_out, L]
    bf16 or None; out may be the residual (in place)."""
    batch, dim_in, L = y.shape
    dim_out = W.shape[0]
    dev = y.device
    _bf16_act("y", y, (batch, dim_in, L), dev)
    _bf16_act("W", W, (dim_out, dim_in), dev)
    _param("bias", bias, (dim_out,), dev)
    if residual is not None:
        _bf16_act("residual", residual, (batch, dim_out, L), dev)
    o = torch.empty(batch, dim_out, L, dtype=torch.bfloat16, device=dev) if out is None else out
    _bf16_act("out", o, (batch, dim_out, L), dev)
    rc = nat.lib.vim_out_proj(batch, dim_in, dim_out, L, nat.VS_BF16, _ptr(y), _ptr(W),
                              _ptr(bias), _ptr(residual), _ptr(o), _stream(dev))
    nat.check("vim_out_proj", rc)
    return o


class VimScanFunction(torch.autograd.Function):
    """vim_scan_bidir for autograd: the forward runs vim_scan_bidir_fwd_saved
    and keeps its saved-state buffer for the backward, which runs
    vim_scan_bidir_grad_saved. The gradients of B and C come back in B's and
    C's dtype (the library sums them in fp32); Dskip and dt_bias given as
    None get no gradient."""

    @staticmethod
    def forward(ctx, u, delta, z, B, C, A, Dskip, dt_bias, delta_softplus=True):
        y, saved = vim_scan_bidir_fwd_saved(u, delta, z, B, C, A, Dskip, dt_bias,
                                            delta_softplus=delta_softplus)
        ctx.save_for_backward(u, delta, z, B, C, A, Dskip, dt_bias, saved)
        ctx.delta_softplus = delta_softplus
        return y

    @staticmethod
    def backward(ctx, dy):
        u, delta, z, B, C, A, Dskip, dt_bias, saved = ctx.saved_tensors
        dy = dy.to(u.dtype).contiguous()
        g = vim_scan_bidir_grad_saved(u, delta, z, B, C, A, Dskip, dt_bias, saved, dy,
                                      delta_softplus=ctx.delta_softplus)
        return (g["du"], g["ddelta"], g["dz"], g["dB"].to(B.dtype), g["dC"].to(C.dtype), g["dA"],
                None if Dskip is None else g["dD"], None if dt_bias is None else g["ddt_bias"], None)


def vim_scan_bidir_autograd(u, delta, z, B, C, A, Dskip=None, dt_bias=None, delta_softplus=True):
    """vim_scan_bidir as a differentiable op (VimScanFunction)."""
    return VimScanFunction.apply(u, delta, z, B, C, A, Dskip, dt_bias, delta_softplus)
