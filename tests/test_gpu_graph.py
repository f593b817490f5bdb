"""The scan entry points allocate nothing and issue only kernel launches, so
a caller can capture them in a HIP graph. Each graph below is replayed
several times, with eager work and synchronisations in between, and every
replay must reproduce the eager call bit for bit."""
import numpy as np
import pytest
import torch

from gpu_util import say, upload
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu

REPLAYS = 4


def replay_and_check(run, eager, what):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = run()
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "%s: replay %d differs from the eager call" % (what, r)
        # eager work between replays
        torch.cuda.synchronize()
        _ = run()
        torch.cuda.synchronize()
    say("  %s: %d replays equal the eager call" % (what, REPLAYS))


@pytest.mark.parametrize("base", [wlm.WORKLOADS[0], wlm.WORKLOADS[1]], ids=["f32", "bf16"])
def test_vim_scan_in_a_graph(base):
    import vision_mamba_selective_amd as vms
    wl = base.with_(batch=2, dim=24, seqlen=197)
    t = upload(wlm.make_inputs(wl, random_A=True, random_D=True))
    ws = torch.empty(max(1, vms.workspace_bytes(0, wl.batch, wl.dim, wl.seqlen, t["u"].dtype)),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty_like(t["u"])

    def run():
        return vms.vim_scan_bidir(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"],
                                  t["dt_bias"], out=y, workspace=ws)

    eager = run().clone()
    torch.cuda.synchronize()
    say("case graph vim %s" % wl.dtype)
    replay_and_check(run, eager, "vim_scan_bidir")


def test_cross_scan_in_a_graph():
    import vision_mamba_selective_amd as vms
    wl = wlm.WORKLOADS[3].with_(batch=2, dim=8, H=13, W=21, seqlen=13 * 21)
    t = upload(wlm.make_inputs(wl, random_A=True, random_D=True))
    ws = torch.empty(vms.workspace_bytes(1, wl.batch, wl.dim, wl.seqlen, t["u"].dtype),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty_like(t["u"])

    def run():
        return vms.vmamba_cross_scan4(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], wl.H, wl.W,
                                      t["Dskip"], t["dt_bias"], out=y, workspace=ws)

    eager = run().clone()
    torch.cuda.synchronize()
    say("case graph cross4")
    replay_and_check(run, eager, "vmamba_cross_scan4")


def test_gradient_in_a_graph():
    """The gradient's three kernels; every output, the fixed-order sums
    included, must repeat bit for bit."""
    import vision_mamba_selective_amd as vms
    wl = wlm.WORKLOADS[1].with_(batch=2, dim=24, seqlen=70)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    t = upload(inp)
    dy = torch.from_numpy(wlm.round_bf16(np.random.default_rng(5).standard_normal(inp.u.shape)
                                         .astype(np.float32))).cuda().to(torch.bfloat16)
    ws = torch.empty(vms.workspace_bytes(3, wl.batch, wl.dim, wl.seqlen, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def run():
        g = vms.vim_scan_bidir_grad(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"],
                                    t["dt_bias"], dy, workspace=ws)
        return torch.cat([g["du"].float().flatten(), g["ddelta"].float().flatten(),
                          g["dz"].float().flatten(), g["dB"].flatten(), g["dC"].flatten(),
                          g["dA"].flatten(), g["dD"].flatten(), g["ddt_bias"].flatten()])

    eager = run().clone()
    torch.cuda.synchronize()
    say("case graph gradient")
    replay_and_check(run, eager, "vim_scan_bidir_grad")


def test_training_pair_in_a_graph():
    """The saving forward and the saved-state gradient captured as one graph
    (a training step of the scan): y and every gradient repeat bit for bit."""
    import vision_mamba_selective_amd as vms
    wl = wlm.WORKLOADS[1].with_(batch=2, dim=24, seqlen=150)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    t = upload(inp)
    dy = torch.from_numpy(wlm.round_bf16(np.random.default_rng(6).standard_normal(inp.u.shape)
                                         .astype(np.float32))).cuda().to(torch.bfloat16)
    saved = torch.empty(vms.workspace_bytes(4, wl.batch, wl.dim, wl.seqlen, torch.bfloat16),
                        dtype=torch.uint8, device="cuda")
    ws = torch.empty(vms.workspace_bytes(5, wl.batch, wl.dim, wl.seqlen, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty_like(t["u"])
    args = (t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"], t["dt_bias"])

    def run():
        vms.vim_scan_bidir_fwd_saved(*args, out=y, saved=saved)
        g = vms.vim_scan_bidir_grad_saved(*args, saved, dy, workspace=ws)
        return torch.cat([y.float().flatten(), g["du"].float().flatten(), g["ddelta"].float().flatten(),
                          g["dz"].float().flatten(), g["dB"].flatten(), g["dC"].flatten(),
                          g["dA"].flatten(), g["dD"].flatten(), g["ddt_bias"].flatten()])

    eager = run().clone()
    torch.cuda.synchronize()
    say("case graph training pair")
    replay_and_check(run, eager, "vim_scan_bidir_fwd_saved + vim_scan_bidir_grad_saved")


def test_out_proj_in_a_graph():
    import vision_mamba_selective_amd as vms
    rng = np.random.default_rng(11)
    bf = lambda a: torch.from_numpy(wlm.round_bf16(a.astype(np.float32))).cuda().to(torch.bfloat16)
    y = bf(rng.standard_normal((2, 96, 197)))
    W = bf(rng.standard_normal((96, 96)) / np.sqrt(96))
    bias = torch.from_numpy(rng.standard_normal(96).astype(np.float32)).cuda()
    res = bf(rng.standard_normal((2, 96, 197)))
    out = torch.empty_like(y)

    def run():
        return vms.vim_out_proj(y, W, bias, res, out=out)

    eager = run().clone()
    torch.cuda.synchronize()
    say("case graph out_proj")
    replay_and_check(run, eager, "vim_out_proj")
