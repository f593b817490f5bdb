"""Seeded random shapes for every scan entry point, checked against the fp64
oracle element by element through the C ABI: sequence lengths around the
16-token blocks and 32-token tiles, channel counts that leave workgroups
partly idle, d_state from 1 to 16, H != W grids for the cross-scan, bf16 and
fp32, with and without the gate and the exact hold, the gradient, and the
training pair (the saving forward's y and the gradient from its saved
states)."""
import numpy as np
import pytest

import oracle
import gpu_util as gu
import test_gpu_conv as tc
import test_gpu_dirs as td
import test_gpu_grad as tg
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu

BASES = [wlm.WORKLOADS[0], wlm.WORKLOADS[1]]
NCASE = 80


@pytest.mark.parametrize("case", range(NCASE))
def test_random_shape(case):
    import vision_mamba_selective_amd as vms
    rng = np.random.default_rng(4242 + case)

    def pick_L():
        r = rng.random()
        if r < 0.5:
            k = int(rng.integers(1, 12))
            return max(1, 16 * k + int(rng.integers(-2, 3)))
        return int(rng.integers(1, 400))

    kind = ["vim", "vim", "cross4", "1d", "conv", "dirs", "grad", "saved"][case % 8]
    base = BASES[int(rng.integers(0, 2))]
    b = int(rng.integers(1, 4))
    d = int(rng.integers(1, 41))
    N = int(rng.choice([1, 4, 8, 12, 15, 16, 16, 16]))
    gate = bool(rng.random() < 0.7)
    zoh = bool(rng.random() < 0.25) and kind not in ("grad", "saved")
    seed = int(rng.integers(0, 1 << 30))
    if kind == "cross4":
        H, W = int(rng.integers(1, 41)), int(rng.integers(1, 41))
        wl = wlm.WORKLOADS[3].with_(batch=b, dim=d, dstate=N, H=H, W=W, seqlen=H * W, gate=gate,
                                    seed=seed, dtype=base.dtype)
    else:
        L = pick_L()
        wl = base.with_(batch=b, dim=d, seqlen=L, dstate=N, gate=gate, seed=seed)
    tag = "%d %s %s b%d d%d L%d N%d gate=%s zoh=%s" % (case, kind, wl.dtype, b, d, wl.seqlen, N, gate, zoh)
    gu.say("case " + tag)
    if kind in ("vim", "cross4"):
        inp = wlm.make_inputs(wl, random_A=True, random_D=True)
        t = gu.upload(inp)
        if kind == "vim":
            y = vms.vim_scan_bidir(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"],
                                   t["dt_bias"], zoh=zoh)
        else:
            y = vms.vmamba_cross_scan4(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], wl.H, wl.W,
                                       t["Dskip"], t["dt_bias"], zoh=zoh)
        ref = oracle.run_inputs(inp, zoh=zoh)
        gu.assert_close(gu.host64(y), ref, wl.dtype, tag)
    elif kind == "1d":
        inp = wlm.make_inputs(wl, random_A=True, random_D=True)
        t = gu.upload(inp)
        rev = bool(rng.random() < 0.5)
        y = vms.s6_scan_1d(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"][0], t["Dskip"][0],
                           t["dt_bias"][0], reverse=rev, zoh=zoh)
        ref = oracle.s6_1d(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A[0], inp.D[0], inp.dt_bias[0],
                           reverse=rev, zoh=zoh)
        gu.assert_close(gu.host64(y), ref, wl.dtype, tag)
    elif kind == "conv":
        inp = wlm.make_inputs(wl, random_A=True, random_D=True)
        w, cb = tc.conv_params(d, seed=seed % 1000, bias=bool(rng.random() < 0.5))
        tt = gu.upload(inp)
        y = vms.vim_scan_bidir_conv(tt["u"], gu.dev(w, gu.torch.float32), gu.dev(cb, gu.torch.float32),
                                    tt["delta"], tt["z"], tt["B"], tt["C"], tt["A"], tt["Dskip"],
                                    tt["dt_bias"], zoh=zoh)
        ref = oracle.vim_conv(inp.u, w, cb, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D, inp.dt_bias,
                              zoh=zoh)
        gu.assert_close(gu.host64(y), ref, wl.dtype, tag)
    elif kind == "dirs":
        x = td.dir_inputs(wl)
        y = gu.host64(td.run(wl, x))
        gu.assert_close(y, td.reference(x), wl.dtype, tag)
    elif kind == "grad":
        inp = wlm.make_inputs(wl, random_A=True, random_D=True)
        dy = tg.upstream(inp, seed=seed % 1000)
        got = tg.run_grad(inp, dy)
        ref = oracle.vim_bidir_grad(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D, inp.dt_bias, dy)
        tg.compare(got, ref, wl.dtype, tag)
    else:
        inp = wlm.make_inputs(wl, random_A=True, random_D=True)
        dy = tg.upstream(inp, seed=seed % 1000)
        t = gu.upload(inp)
        args = (t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"], t["dt_bias"])
        y, saved = vms.vim_scan_bidir_fwd_saved(*args)
        got = vms.vim_scan_bidir_grad_saved(*args, saved, gu.dev(dy, gu.torch_dtype(wl)))
        gu.assert_close(gu.host64(y), oracle.run_inputs(inp), wl.dtype, tag + " y")
        ref = oracle.vim_bidir_grad(inp.u, inp.delta, inp.z, inp.B, inp.C, inp.A, inp.D, inp.dt_bias, dy)
        tg.compare(got, ref, wl.dtype, tag)
