"""GPU parity of the Vim bidirectional scan and the single-direction scan
against the fp64 oracle, element by element, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (STRICT, assert_close, host64, run_gpu, say, stable_without_softplus, strict_bound,
                      strict_err, upload)
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu

VIM_F32 = wlm.WORKLOADS[0]
VIM_BF16 = wlm.WORKLOADS[1]


def check(inp, what, **kw):
    say("case %s %s" % (what, inp.wl))
    y = host64(run_gpu(inp, **kw))
    ref = oracle.run_inputs(inp)
    err = assert_close(y, ref, inp.wl.dtype, what)
    say("  max rel err %.3g" % err)
    return y, ref


# ---- small shapes the oracle finishes at once: several tiles, ragged tails
SMALL = [
    # batch, dim, L, dstate
    (1, 1, 1, 16),
    (1, 3, 5, 16),
    (2, 13, 37, 16),
    (1, 8, 197, 16),
    (3, 10, 64, 8),
    (1, 9, 33, 1),
    (2, 17, 31, 16),
    (1, 16, 32, 16),
    (1, 7, 255, 12),
]


@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_vim_small(shape, base):
    b, d, L, N = shape
    wl = base.with_(batch=b, dim=d, seqlen=L, dstate=N, seed=sum(shape) * 7 + len(SMALL))
    check(wlm.make_inputs(wl, random_A=True, random_D=True), "small%s" % (shape,))


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_vim_no_gate_and_no_softplus(base):
    wl = base.with_(batch=2, dim=11, seqlen=70, gate=False)
    inp = wlm.make_inputs(wl, random_D=True)
    check(inp, "no gate")
    stable_without_softplus(inp)
    say("case softplus off")
    y = host64(run_gpu(inp, delta_softplus=False))
    ref = oracle.vim_bidir(inp.u, inp.delta, None, inp.B, inp.C, inp.A, inp.D, inp.dt_bias,
                           delta_softplus=False)
    assert_close(y, ref, wl.dtype, "softplus off")


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_vim_scan_only_strict(base):
    """D = 0 and no gate: the output is the scan term alone, so an indexing
    slip cannot hide under the D*u skip."""
    wl = base.with_(batch=2, dim=24, seqlen=300, gate=False)
    inp = wlm.make_inputs(wl, random_A=True)
    inp.D[:] = 0.0
    say("case scan-only strict %s" % wl.dtype)
    y = host64(run_gpu(inp))
    ref = oracle.run_inputs(inp)
    err, rms = strict_err(y, ref, wl.dtype)
    say("  max (|dy| - output rounding) / rms = %.3g (rms %.3g)" % (err, rms))
    assert err <= STRICT[wl.dtype]


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_vim_delta_zero_is_exact(base):
    """delta = 0 with softplus off and no bias: the state stays 0 and
    y = D_f u + D_b u = 2u exactly."""
    wl = base.with_(batch=2, dim=9, seqlen=50, gate=False)
    inp = wlm.make_inputs(wl)
    inp.delta[:] = 0.0
    t = upload(inp)
    t["dt_bias"] = None
    import vision_mamba_selective_amd as vms
    say("case delta zero")
    y = vms.vim_scan_bidir(t["u"], t["delta"], None, t["B"], t["C"], t["A"], t["Dskip"], None,
                           delta_softplus=False)
    assert torch.equal(y, 2 * t["u"])


# The forward and backward rows of a channel hand each other their partial
# sums through LDS when a workgroup's 8 channels x L fp32 entries and two
# 16-entry guards fit in 8 KB (L <= 252), through global memory beyond.
PART_EDGE = [(252, "LDS"), (253, "global"), (197, "LDS"), (17, "LDS")]


@pytest.mark.parametrize("case", PART_EDGE, ids=["%d-%s" % c for c in PART_EDGE])
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_vim_either_side_of_the_lds_partial_limit(case, base):
    L, where = case
    assert (8 * L + 32) * 4 <= 8192 if where == "LDS" else (8 * L + 32) * 4 > 8192
    wl = base.with_(batch=2, dim=11, seqlen=L, seed=500 + L)
    check(wlm.make_inputs(wl, random_A=True, random_D=True), "partial sums in %s, L %d" % (where, L))
    # scan term alone (D = 0, no gate): a partial sum handed to the wrong
    # token or lane cannot hide under the skip term
    wl = wl.with_(gate=False)
    inp = wlm.make_inputs(wl, random_A=True)
    inp.D[:] = 0.0
    say("case partial sums in %s, strict, L %d" % (where, L))
    y = host64(run_gpu(inp))
    err, rms = strict_err(y, oracle.run_inputs(inp), wl.dtype)
    say("  max (|dy| - output rounding) / rms = %.3g (rms %.3g)" % (err, rms))
    assert err <= STRICT[wl.dtype]


def test_vim_repeatable_and_in_bounds():
    """Two runs give identical bits; nothing outside y is written."""
    wl = VIM_BF16.with_(batch=3, dim=21, seqlen=111)
    inp = wlm.make_inputs(wl)
    t = upload(inp)
    n = wl.batch * wl.dim * wl.seqlen
    guard = 4096
    canary = torch.full((n + 2 * guard,), 7.25, dtype=torch.bfloat16, device="cuda")
    out = canary[guard:guard + n].view(wl.batch, wl.dim, wl.seqlen)
    say("case repeat/canary")
    y1 = run_gpu(inp, t, out=out).clone()
    y2 = run_gpu(inp, t)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.all(canary[:guard] == 7.25) and torch.all(canary[guard + n:] == 7.25)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_s6_1d(reverse, base):
    import vision_mamba_selective_amd as vms
    wl = base.with_(batch=2, dim=19, seqlen=99)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    t = upload(inp)
    say("case 1d reverse=%s" % reverse)
    y = host64(vms.s6_scan_1d(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"][0],
                              t["Dskip"][0], t["dt_bias"][0], reverse=reverse))
    ref = oracle.s6_1d(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A[0], inp.D[0], inp.dt_bias[0],
                       reverse=reverse)
    assert_close(y, ref, wl.dtype, "1d")


# ---- the workloads at full size, in the launch configuration the benchmark
# times. Every element of y is compared with the oracle, which takes about a
# second per workload on the host's cores.
@pytest.mark.parametrize("idx", [0, 1, 2, 4, 5])
def test_vim_workload_full_size(idx):
    wl = wlm.WORKLOADS[idx]
    say("case workload %d %s" % (idx, wl.name))
    inp = wlm.make_inputs(wl)
    y = host64(run_gpu(inp))
    ref = oracle.run_inputs(inp)
    err = assert_close(y, ref, wl.dtype, wl.name)
    say("  %s max rel err %.3g over all %d outputs" % (wl.name, err, y.size))


@pytest.mark.parametrize("idx", [2, 4])
def test_vim_scan_only_strict_full_length(idx):
    """The strict scan-only check (D = 0, no gate, random A) at the full
    sequence lengths of Vim-S 1024^2 and Vim-B 2048^2: a carry error over
    thousands of steps cannot hide under the D*u term here."""
    wl = wlm.WORKLOADS[idx].with_(gate=False)
    say("case scan-only strict full length %s" % wl.name)
    inp = wlm.make_inputs(wl, random_A=True)
    inp.D[:] = 0.0
    y = host64(run_gpu(inp))
    ref = oracle.run_inputs(inp)
    err, rms = strict_err(y, ref, wl.dtype)
    say("  max (|dy| - output rounding) / rms = %.3g (rms %.3g, L %d)" % (err, rms, wl.seqlen))
    assert err <= strict_bound(wl.dtype, wl.seqlen)
