"""GPU parity of vim_scan_bidir_conv (the Vim scan with the block's conv1d +
SiLU front end fused into its token loads) against the fp64 oracle's
vim_conv, element by element, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (STRICT, assert_close, dev, host64, say, stable_without_softplus,
                      strict_err, torch_dtype, upload)
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu

VIM_F32 = wlm.WORKLOADS[0]
VIM_BF16 = wlm.WORKLOADS[1]


def conv_params(dim, seed, bias=True):
    rng = np.random.default_rng(seed)
    w = (0.6 * rng.standard_normal((2, dim, 3))).astype(np.float32)
    b = (0.2 * rng.standard_normal((2, dim))).astype(np.float32) if bias else None
    return w, b


def run(inp, w, b, delta_softplus=True):
    import vision_mamba_selective_amd as vms
    t = upload(inp)
    cw = dev(w, torch.float32)
    cb = dev(b, torch.float32)
    return vms.vim_scan_bidir_conv(t["u"], cw, cb, t["delta"], t["z"], t["B"], t["C"], t["A"],
                                   t["Dskip"], t["dt_bias"], delta_softplus=delta_softplus)


def reference(inp, w, b, delta_softplus=True):
    return oracle.vim_conv(inp.u, w, b, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D,
                           inp.dt_bias, delta_softplus=delta_softplus)


SMALL = [
    # batch, dim, L, dstate
    (1, 1, 1, 16),
    (1, 3, 2, 16),
    (2, 13, 37, 16),
    (1, 8, 197, 16),
    (3, 10, 64, 8),
    (2, 17, 31, 16),
    (1, 7, 255, 12),
]


@pytest.mark.parametrize("bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_conv_small(shape, base, bias):
    b_, d, L, N = shape
    wl = base.with_(batch=b_, dim=d, seqlen=L, dstate=N, seed=sum(shape) * 13 + bias)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    w, cb = conv_params(d, seed=sum(shape) + 5, bias=bias)
    say("case conv small%s bias=%s %s" % (shape, bias, wl.dtype))
    y = host64(run(inp, w, cb))
    err = assert_close(y, reference(inp, w, cb), wl.dtype, "conv small")
    say("  max rel err %.3g" % err)


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_conv_no_gate_no_softplus(base):
    wl = base.with_(batch=2, dim=11, seqlen=70, gate=False)
    inp = wlm.make_inputs(wl, random_D=True)
    stable_without_softplus(inp)
    w, cb = conv_params(11, seed=9)
    say("case conv no gate, softplus off")
    y = host64(run(inp, w, cb, delta_softplus=False))
    assert_close(y, reference(inp, w, cb, delta_softplus=False), wl.dtype, "conv plain")


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_conv_scan_only_strict(base):
    """D = 0 and no gate: the output is the two scan terms alone."""
    wl = base.with_(batch=2, dim=24, seqlen=300, gate=False)
    inp = wlm.make_inputs(wl, random_A=True)
    inp.D[:] = 0.0
    w, cb = conv_params(24, seed=10)
    say("case conv scan-only strict %s" % wl.dtype)
    y = host64(run(inp, w, cb))
    err, rms = strict_err(y, reference(inp, w, cb), wl.dtype)
    say("  max (|dy| - output rounding) / rms = %.3g (rms %.3g)" % (err, rms))
    assert err <= STRICT[wl.dtype]


def test_conv_identity_taps_equal_plain_scan_of_silu():
    """Taps (0, 1, 0) without bias make both branches' u = silu(x): the
    result is the plain bidirectional scan of silu(x) (both sides checked
    against the oracle)."""
    import vision_mamba_selective_amd as vms
    wl = VIM_F32.with_(batch=2, dim=9, seqlen=45)
    inp = wlm.make_inputs(wl)
    w = np.zeros((2, 9, 3), np.float32)
    w[..., 1] = 1.0
    say("case conv identity taps")
    y = host64(run(inp, w, None))
    ref = reference(inp, w, None)
    assert_close(y, ref, wl.dtype, "identity taps")
    t = upload(inp)
    su = torch.nn.functional.silu(t["u"])
    y2 = host64(vms.vim_scan_bidir(su, t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"],
                                   t["dt_bias"]))
    assert_close(y2, ref, wl.dtype, "plain scan of silu(x)")


def test_conv_workload_full_size():
    """The Vim-S 1024x1024 workload with the front end, at full size; every
    element of y is compared with the oracle."""
    wl = wlm.WORKLOADS[2]
    say("case conv workload %s" % wl.name)
    inp = wlm.make_inputs(wl)
    w, cb = conv_params(wl.dim, seed=2024)
    y = host64(run(inp, w, cb))
    err = assert_close(y, reference(inp, w, cb), wl.dtype, "conv full size")
    say("  max rel err %.3g over all %d outputs" % (err, y.size))
    assert torch_dtype(wl) == torch.bfloat16
