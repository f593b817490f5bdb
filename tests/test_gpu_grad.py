"""GPU parity of vim_scan_bidir_grad (reverse-mode gradient of the Vim scan)
against the fp64 oracle's vim_bidir_grad, element by element, through the C
ABI.

Tolerances (|g - g_ref| <= tol * (1 + |g_ref|)):
  * du, ddelta, dz are written in the input dtype: 1e-4 for fp32 (the
    forward's bound; the adjoint recurrence runs in fp32 like the forward
    one) and 2e-2 for bf16 (the final bf16 rounding dominates, as for y);
  * dB, dC, dA, dD, ddt_bias are fp32 sums over channels, batch rows and
    steps, taken in a fixed order: 2e-4 for either input dtype, since the
    inputs are exact in fp32 and only the fp32 accumulation differs (the
    per-element sums have at most a few thousand terms)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_finite, dev, host64, say, stable_without_softplus, torch_dtype, upload
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu

VIM_F32 = wlm.WORKLOADS[0]
VIM_BF16 = wlm.WORKLOADS[1]
PER_TOKEN = ("du", "ddelta", "dz")
SUMMED = ("dB", "dC", "dA", "dD", "ddt_bias")
TOL_TOKEN = {wlm.F32: 1e-4, wlm.BF16: 2e-2}
TOL_SUM = 2e-4


def upstream(inp, seed):
    g = np.random.default_rng(seed).standard_normal(inp.u.shape).astype(np.float32)
    return wlm.round_bf16(g) if inp.wl.dtype == wlm.BF16 else g


def run_grad(inp, dy, delta_softplus=True):
    import vision_mamba_selective_amd as vms
    t = upload(inp)
    return vms.vim_scan_bidir_grad(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"],
                                   t["Dskip"], t["dt_bias"], dev(dy, torch_dtype(inp.wl)),
                                   delta_softplus=delta_softplus)


def compare(got, ref, dtype, what, keys=PER_TOKEN + SUMMED):
    errs = {}
    for k in keys:
        if got.get(k) is None:
            assert not np.any(ref[k]), k
            continue
        g = host64(got[k])
        assert_finite(g, ref[k], "%s %s" % (what, k))
        tol = TOL_TOKEN[dtype] if k in PER_TOKEN else TOL_SUM
        bad = np.abs(g - ref[k]) > tol * (1.0 + np.abs(ref[k]))
        errs[k] = float(np.max(np.abs(g - ref[k]) / (1.0 + np.abs(ref[k]))))
        if bad.any():
            idx = np.argwhere(bad)[:4]
            raise AssertionError("%s %s: %d beyond %.0e (max rel %.3g); at %s got %s ref %s" % (
                what, k, int(bad.sum()), tol, errs[k], idx.tolist(),
                g[tuple(idx.T)].tolist(), ref[k][tuple(idx.T)].tolist()))
    say("  " + " ".join("%s %.2g" % kv for kv in errs.items()))


SMALL = [
    # batch, dim, L, dstate
    (1, 1, 1, 16),
    (1, 3, 5, 16),
    (2, 13, 37, 16),
    (1, 8, 197, 16),
    (3, 10, 64, 8),
    (2, 17, 31, 16),
    (1, 7, 255, 12),
]


@pytest.mark.parametrize("gate", [True, False], ids=["gated", "plain"])
@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_grad_small(shape, base, gate):
    b_, d, L, N = shape
    wl = base.with_(batch=b_, dim=d, seqlen=L, dstate=N, gate=gate, seed=sum(shape) * 17 + gate)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    dy = upstream(inp, seed=sum(shape))
    say("case grad small%s gate=%s %s" % (shape, gate, wl.dtype))
    got = run_grad(inp, dy)
    ref = oracle.vim_bidir_grad(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D,
                                inp.dt_bias, dy)
    compare(got, ref, wl.dtype, "grad small")


# batch x ceil(dim / 24) >= 256: the launcher takes 24-channel workgroups
# (768 threads); dims that are not multiples of 24 leave idle channels
WIDE = [
    # batch, dim, L, dstate
    (256, 20, 37, 16),
    (128, 50, 45, 12),
]


@pytest.mark.parametrize("shape", WIDE)
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_grad_wide_workgroups(shape, base):
    b_, d, L, N = shape
    wl = base.with_(batch=b_, dim=d, seqlen=L, dstate=N, seed=sum(shape) * 19)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    dy = upstream(inp, seed=sum(shape) + 1)
    say("case grad wide%s %s" % (shape, wl.dtype))
    got = run_grad(inp, dy)
    ref = oracle.vim_bidir_grad(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D,
                                inp.dt_bias, dy)
    compare(got, ref, wl.dtype, "grad wide")


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_grad_softplus_off(base):
    wl = base.with_(batch=2, dim=11, seqlen=70)
    inp = wlm.make_inputs(wl, random_D=True)
    stable_without_softplus(inp)
    dy = upstream(inp, seed=3)
    say("case grad softplus off %s" % wl.dtype)
    got = run_grad(inp, dy, delta_softplus=False)
    ref = oracle.vim_bidir_grad(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D,
                                inp.dt_bias, dy, delta_softplus=False)
    compare(got, ref, wl.dtype, "grad softplus off")


def test_grad_outputs_are_repeatable():
    """du, ddelta and dz have one writer per element, and dB, dC, dA, dD and
    ddt_bias are summed in a fixed order: identical bits across calls."""
    wl = VIM_BF16.with_(batch=2, dim=16, seqlen=100)
    inp = wlm.make_inputs(wl)
    dy = upstream(inp, seed=4)
    say("case grad repeatable")
    a = run_grad(inp, dy)
    b = run_grad(inp, dy)
    for k in PER_TOKEN + SUMMED:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("idx", [1, 2, 5])
def test_grad_workload_full_size(idx):
    """The Vim-S workloads at full size against the full oracle gradient
    (every channel contributes to dB and dC)."""
    wl = wlm.WORKLOADS[idx]
    inp = wlm.make_inputs(wl)
    dy = upstream(inp, seed=100 + idx)
    say("case grad workload %s" % wl.name)
    got = run_grad(inp, dy)
    torch.cuda.synchronize()
    ref = oracle.vim_bidir_grad(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D,
                                inp.dt_bias, dy)
    compare(got, ref, wl.dtype, "grad " + wl.name)
