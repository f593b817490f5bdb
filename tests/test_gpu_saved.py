"""GPU parity of the training pair vim_scan_bidir_fwd_saved and
vim_scan_bidir_grad_saved, through the C ABI.

  * y of the saving forward is the unchunked vim_scan_bidir's y bit for bit
    (the same arithmetic in the same order; vim_scan_bidir itself may cut
    short grids into chunks, whose carry combine rounds differently) and the
    oracle's to the forward tolerance;
  * the gradient read from the saved buffer is vim_scan_bidir_grad's bit
    for bit (which recomputes the same forward pass into its workspace) and
    the oracle's vim_bidir_grad to the gradient tolerances;
over ragged shapes, both dtypes, with and without the gate and softplus,
both gradient workgroup widths, one saved buffer reused for two upstream
gradients, and the Vim-S 1024^2 workload at full size."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, host64, say, stable_without_softplus, torch_dtype, upload
from test_gpu_grad import PER_TOKEN, SUMMED, compare, upstream
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu

VIM_F32 = wlm.WORKLOADS[0]
VIM_BF16 = wlm.WORKLOADS[1]


def pair(t, dy_t, delta_softplus=True):
    """(y, saved-state gradient) of the training pair, and (y, gradient) of
    the plain forward and the recomputing gradient, on the same inputs."""
    import vision_mamba_selective_amd as vms
    args = (t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"], t["dt_bias"])
    y_s, saved = vms.vim_scan_bidir_fwd_saved(*args, delta_softplus=delta_softplus)
    g_s = vms.vim_scan_bidir_grad_saved(*args, saved, dy_t, delta_softplus=delta_softplus)
    y_p = vms.vim_scan_bidir_chunked(*args, chunks=1, delta_softplus=delta_softplus)
    g_p = vms.vim_scan_bidir_grad(*args, dy_t, delta_softplus=delta_softplus)
    return y_s, g_s, y_p, g_p, saved


def same_bits(g_s, g_p, what):
    for k in PER_TOKEN + SUMMED:
        if g_p[k] is None:
            assert g_s[k] is None, (what, k)
            continue
        assert torch.equal(g_s[k], g_p[k]), (what, k)


SHAPES = [
    # batch, dim, L, dstate
    (1, 1, 1, 16),
    (2, 13, 37, 16),
    (1, 8, 197, 16),
    (3, 10, 64, 8),
    (2, 9, 1000, 16),
]


@pytest.mark.parametrize("gate", [True, False], ids=["gated", "plain"])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_saved_pair_matches_plain_calls_and_oracle(shape, base, gate):
    b_, d, L, N = shape
    wl = base.with_(batch=b_, dim=d, seqlen=L, dstate=N, gate=gate, seed=sum(shape) * 23 + gate)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    dy = upstream(inp, seed=sum(shape) + 5)
    say("case saved pair %s gate=%s %s" % (shape, gate, wl.dtype))
    t = upload(inp)
    y_s, g_s, y_p, g_p, _ = pair(t, dev(dy, torch_dtype(wl)))
    assert torch.equal(y_s, y_p)
    same_bits(g_s, g_p, "saved pair")
    assert_close(host64(y_s), oracle.run_inputs(inp), wl.dtype, "saving forward y")
    ref = oracle.vim_bidir_grad(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D, inp.dt_bias, dy)
    compare(g_s, ref, wl.dtype, "saved gradient")


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_saved_pair_softplus_off(base):
    wl = base.with_(batch=2, dim=11, seqlen=70)
    inp = stable_without_softplus(wlm.make_inputs(wl, random_D=True))
    dy = upstream(inp, seed=41)
    say("case saved pair softplus off %s" % wl.dtype)
    t = upload(inp)
    y_s, g_s, y_p, g_p, _ = pair(t, dev(dy, torch_dtype(wl)), delta_softplus=False)
    assert torch.equal(y_s, y_p)
    same_bits(g_s, g_p, "softplus off")
    ref = oracle.vim_bidir_grad(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D, inp.dt_bias, dy,
                                delta_softplus=False)
    compare(g_s, ref, wl.dtype, "saved gradient, softplus off")


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_saved_pair_wide_workgroups(base):
    """batch x ceil(dim / 24) >= 256: the gradient takes 24-channel
    workgroups; dim 50 leaves idle channels in the last one."""
    wl = base.with_(batch=128, dim=50, seqlen=45, seed=611)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    dy = upstream(inp, seed=612)
    say("case saved pair wide %s" % wl.dtype)
    t = upload(inp)
    y_s, g_s, y_p, g_p, _ = pair(t, dev(dy, torch_dtype(wl)))
    assert torch.equal(y_s, y_p)
    same_bits(g_s, g_p, "wide")


def test_one_saved_buffer_serves_two_backward_calls():
    """The saved buffer is read only: two upstream gradients on one buffer
    each give vim_scan_bidir_grad's result."""
    import vision_mamba_selective_amd as vms
    wl = VIM_BF16.with_(batch=2, dim=12, seqlen=300, seed=77)
    inp = wlm.make_inputs(wl, random_A=True)
    t = upload(inp)
    args = (t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"], t["dt_bias"])
    _, saved = vms.vim_scan_bidir_fwd_saved(*args)
    keep = saved.clone()
    for seed in (1, 2):
        dy_t = dev(upstream(inp, seed=seed), torch.bfloat16)
        say("case saved reuse seed %d" % seed)
        same_bits(vms.vim_scan_bidir_grad_saved(*args, saved, dy_t), vms.vim_scan_bidir_grad(*args, dy_t),
                  "reuse %d" % seed)
    torch.cuda.synchronize()
    assert torch.equal(saved, keep)


def test_vim_s_1024_saved_pair():
    """The Vim-S 1024^2 workload (batch 8, 768 channels, 4,097 tokens) at full
    size: the pair against the plain calls, bit for bit (the plain gradient
    is checked against the oracle at this size in test_gpu_grad.py)."""
    wl = wlm.WORKLOADS[2]
    inp = wlm.make_inputs(wl)
    dy = upstream(inp, seed=9)
    say("case saved pair vim_s_1024")
    t = upload(inp)
    y_s, g_s, y_p, g_p, _ = pair(t, dev(dy, torch_dtype(wl)))
    assert torch.equal(y_s, y_p)
    same_bits(g_s, g_p, "vim_s_1024")
    for k in PER_TOKEN + SUMMED:
        assert torch.isfinite(g_s[k].float()).all(), k


@pytest.mark.parametrize("gate", [True, False], ids=["gated", "plain"])
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_autograd_function(base, gate):
    """VimScanFunction: y.backward(dy) leaves the saved-state gradient in
    every input's .grad (B and C in their dtype), the same bits as the
    library calls, and the oracle's gradient to the gradient tolerances."""
    import vision_mamba_selective_amd as vms
    wl = base.with_(batch=2, dim=10, seqlen=150, gate=gate, seed=321 + gate)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    dy = upstream(inp, seed=17)
    t = upload(inp)
    leaves = {k: (v.clone().requires_grad_(True) if v is not None else None) for k, v in t.items()}
    say("case autograd %s gate=%s" % (wl.dtype, gate))
    y = vms.vim_scan_bidir_autograd(leaves["u"], leaves["delta"], leaves["z"], leaves["B"], leaves["C"],
                                    leaves["A"], leaves["Dskip"], leaves["dt_bias"])
    dy_t = dev(dy, torch_dtype(wl))
    y.backward(dy_t)
    args = (t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"], t["dt_bias"])
    y_p, saved = vms.vim_scan_bidir_fwd_saved(*args)
    g = vms.vim_scan_bidir_grad_saved(*args, saved, dy_t)
    assert torch.equal(y.detach(), y_p)
    names = {"u": "du", "delta": "ddelta", "z": "dz", "A": "dA", "Dskip": "dD", "dt_bias": "ddt_bias"}
    for leaf, key in names.items():
        if leaves[leaf] is None:
            continue
        assert torch.equal(leaves[leaf].grad, g[key]), leaf
    for leaf, key in (("B", "dB"), ("C", "dC")):
        assert leaves[leaf].grad.dtype == t[leaf].dtype
        assert torch.equal(leaves[leaf].grad, g[key].to(t[leaf].dtype)), leaf
    ref = oracle.vim_bidir_grad(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D, inp.dt_bias, dy)
    got = {names[k]: leaves[k].grad for k in names if leaves[k] is not None}
    got.update(dB=g["dB"], dC=g["dC"])
    if not gate:
        got["dz"] = None
    compare(got, ref, wl.dtype, "autograd")
