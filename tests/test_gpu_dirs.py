"""GPU parity of vim_scan_bidir_dirs (the Vim scan with per-direction u,
delta, B and C) against the fp64 oracle's vim_dirs, element by element,
through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, host64, say, torch_dtype, upload
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu

VIM_F32 = wlm.WORKLOADS[0]
VIM_BF16 = wlm.WORKLOADS[1]


def dir_inputs(wl, random=True):
    """Copy 0 from the workload's own draw, copy 1 from a second draw (seed
    + 1): u, delta [2, batch, dim, L]; B, C [batch, 2, dstate, L]; z, A, D and
    dt_bias from the first draw."""
    a = wlm.make_inputs(wl, random_A=random, random_D=random)
    b = wlm.make_inputs(wl, seed=wl.seed + 1)
    return dict(u=np.stack([a.u, b.u]), delta=np.stack([a.delta, b.delta]), z=a.z,
                B=np.stack([a.B, b.B], axis=1), C=np.stack([a.C, b.C], axis=1), A=a.A, D=a.D,
                dt_bias=a.dt_bias)


def run(wl, x, delta_softplus=True):
    import vision_mamba_selective_amd as vms
    dt = torch_dtype(wl)
    return vms.vim_scan_bidir_dirs(dev(x["u"], dt), dev(x["delta"], dt), dev(x["z"], dt),
                                   dev(x["B"], dt), dev(x["C"], dt), dev(x["A"], torch.float32),
                                   dev(x["D"], torch.float32), dev(x["dt_bias"], torch.float32),
                                   delta_softplus=delta_softplus)


def reference(x, delta_softplus=True):
    return oracle.vim_dirs(x["u"], x["delta"], x["z"], x["B"], x["C"], x["A"], x["D"],
                           x["dt_bias"], delta_softplus=delta_softplus)


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


@pytest.mark.parametrize("gate", [True, False], ids=["gated", "plain"])
@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_dirs_small(shape, base, gate):
    b_, d, L, N = shape
    wl = base.with_(batch=b_, dim=d, seqlen=L, dstate=N, gate=gate, seed=sum(shape) * 23 + gate)
    x = dir_inputs(wl)
    say("case dirs small%s gate=%s %s" % (shape, gate, wl.dtype))
    y = host64(run(wl, x))
    err = assert_close(y, reference(x), wl.dtype, "dirs small")
    say("  max rel err %.3g" % err)


def test_dirs_identical_copies_equal_shared_scan():
    """Both copies equal: the result is vim_scan_bidir's, bit for bit."""
    import vision_mamba_selective_amd as vms
    wl = VIM_BF16.with_(batch=2, dim=24, seqlen=300)
    inp = wlm.make_inputs(wl)
    t = upload(inp)
    say("case dirs identical copies")
    y_shared = vms.vim_scan_bidir(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"],
                                  t["dt_bias"])
    y_dirs = vms.vim_scan_bidir_dirs(torch.stack([t["u"], t["u"]]).contiguous(),
                                     torch.stack([t["delta"], t["delta"]]).contiguous(), t["z"],
                                     torch.stack([t["B"], t["B"]], 1).contiguous(),
                                     torch.stack([t["C"], t["C"]], 1).contiguous(), t["A"],
                                     t["Dskip"], t["dt_bias"])
    assert torch.equal(y_shared, y_dirs)


def test_dirs_workload_full_size():
    """Vim-S 1024x1024 with per-direction inputs at full size; every element
    of y is compared with the oracle."""
    wl = wlm.WORKLOADS[2]
    x = dir_inputs(wl, random=False)
    say("case dirs workload %s" % wl.name)
    y = host64(run(wl, x))
    err = assert_close(y, reference(x), wl.dtype, "dirs full size")
    say("  max rel err %.3g over all %d outputs" % (err, y.size))
