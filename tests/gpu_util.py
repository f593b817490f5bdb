"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP path,
compare with the oracle."""
import sys

import numpy as np
import torch

from vision_mamba_selective_amd import workloads as wlm

#: element-wise bound |y - y_ref| <= TOL * (1 + |y_ref|)
TOL = {wlm.F32: 1e-4, wlm.BF16: 2e-2}
#: strict scan-only diagnostic (D = 0, no gate), derived from the arithmetic:
#: |y - y_ref| <= half_ulp(y_ref) + STRICT[dtype] * rms(y_ref), where half_ulp
#: is the final round-to-nearest of the output (0 for fp32 output: its
#: rounding is below the fp32 arithmetic error) and STRICT bounds the fp32
#: arithmetic of the scan relative to its typical size.
STRICT = {wlm.F32: 1e-5, wlm.BF16: 2e-5}
_SIG_BITS = {wlm.F32: None, wlm.BF16: 8}
#: sequence length at which STRICT was set
_STRICT_L = 300


def strict_bound(dtype, L):
    """STRICT for a sequence of L steps: each step rounds the state (the FMA
    and the hardware exp2, about 2^-24 relative each) and those errors add up
    over the steps the state remembers, like a random walk, so the bound grows
    as sqrt(L) past the length at which STRICT was set."""
    return STRICT[dtype] * max(1.0, (L / _STRICT_L) ** 0.5)


def half_ulp(ref, dtype):
    bits = _SIG_BITS[dtype]
    if bits is None:
        return np.zeros_like(ref)
    _, e = np.frexp(np.abs(ref))           # |ref| = m 2^e, m in [0.5, 1)
    return np.ldexp(1.0, e - 1 - bits)


def strict_err(y, ref, dtype):
    assert_finite(y, ref, "strict")
    rms = float(np.sqrt(np.mean(ref ** 2)))
    excess = np.abs(y - ref) - half_ulp(ref, dtype)
    return float(np.max(excess)) / rms, rms


def stable_without_softplus(inp):
    """Make delta_raw + dt_bias positive (0.2 |delta_raw| + 0.05), so that the
    scan stays bounded when softplus is off; delta is re-rounded to the input
    dtype so that both sides see the same values."""
    d = np.abs(inp.delta) * np.float32(0.2)
    inp.delta = wlm.round_bf16(d) if inp.wl.dtype == wlm.BF16 else d.astype(np.float32)
    inp.dt_bias = np.full_like(inp.dt_bias, 0.05)
    return inp


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(wl):
    return torch.bfloat16 if wl.dtype == wlm.BF16 else torch.float32


def dev(a, dtype, device="cuda"):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(dtype)


def upload(inp, device="cuda"):
    dt = torch_dtype(inp.wl)
    return dict(u=dev(inp.u, dt, device), delta=dev(inp.delta, dt, device),
                z=dev(inp.z, dt, device), B=dev(inp.B, dt, device), C=dev(inp.C, dt, device),
                A=dev(inp.A, torch.float32, device), Dskip=dev(inp.D, torch.float32, device),
                dt_bias=dev(inp.dt_bias, torch.float32, device))


def run_gpu(inp, t=None, delta_softplus=True, out=None):
    """Run the workload's entry point on the GPU; returns the torch output."""
    import vision_mamba_selective_amd as vms
    t = t or upload(inp)
    wl = inp.wl
    if wl.kind == "vim":
        return vms.vim_scan_bidir(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"],
                                  t["dt_bias"], delta_softplus=delta_softplus, out=out)
    return vms.vmamba_cross_scan4(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], wl.H,
                                  wl.W, t["Dskip"], t["dt_bias"], delta_softplus=delta_softplus,
                                  out=out)


def host64(y):
    return y.float().cpu().numpy().astype(np.float64)


def rel_err(y, ref):
    return float(np.max(np.abs(y - ref) / (1.0 + np.abs(ref))))


def assert_finite(y, ref, what=""):
    """Both sides must be finite: comparisons with NaN are false, so a
    non-finite result would otherwise pass every tolerance test."""
    if not np.all(np.isfinite(ref)):
        raise AssertionError("%s: the reference holds non-finite values" % what)
    if not np.all(np.isfinite(y)):
        raise AssertionError("%s: %d non-finite outputs" % (what, int(np.sum(~np.isfinite(y)))))


def assert_close(y, ref, dtype, what=""):
    assert_finite(y, ref, what)
    err = rel_err(y, ref)
    bad = np.abs(y - ref) > TOL[dtype] * (1.0 + np.abs(ref))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d elements beyond tolerance (max rel %.3g); first %s: got %s "
                             "ref %s" % (what, int(bad.sum()), err, idx.tolist(),
                                         y[tuple(idx.T)].tolist(), ref[tuple(idx.T)].tolist()))
    return err
