"""vim_scan_bidir_noalloc, the entry point that allocates nothing (its merge
buffer is the library's static device array), against vim_scan_bidir with a
caller workspace: two calls in a row through the C ABI, the second with a
smaller input, each to the parity bar of the scan and against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close, host64, say, torch_dtype, upload
from vision_mamba_selective_amd import _native as nat
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def call_noalloc(wl, t, y):
    dt = nat.VS_BF16 if wl.dtype == wlm.BF16 else nat.VS_F32
    rc = nat.lib.vim_scan_bidir_noalloc(
        wl.batch, wl.dim, wl.dstate, wl.seqlen, dt, ptr(t["u"]), ptr(t["delta"]), ptr(t["z"]),
        ptr(t["B"]), ptr(t["C"]), ptr(t["A"]), ptr(t["Dskip"]), ptr(t["dt_bias"]), 1, ptr(y),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    nat.check("vim_scan_bidir_noalloc", rc)


def call_with_workspace(wl, t, y):
    dt = nat.VS_BF16 if wl.dtype == wlm.BF16 else nat.VS_F32
    need = nat.lib.vs_workspace_bytes(nat.VS_OP_VIM_BIDIR, wl.batch, wl.dim, wl.seqlen, dt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    rc = nat.lib.vim_scan_bidir(
        wl.batch, wl.dim, wl.dstate, wl.seqlen, dt, ptr(t["u"]), ptr(t["delta"]), ptr(t["z"]),
        ptr(t["B"]), ptr(t["C"]), ptr(t["A"]), ptr(t["Dskip"]), ptr(t["dt_bias"]), 1, ptr(y),
        ptr(ws) if need else None, need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    nat.check("vim_scan_bidir", rc)


@pytest.mark.parametrize("base", [wlm.WORKLOADS[0], wlm.WORKLOADS[2]], ids=["f32", "bf16"])
def test_noalloc_matches_the_workspace_entry_point(base):
    # the second call is smaller than the first, so it reads a buffer that
    # still holds the first call's sums
    shapes = [(3, 40, 1000), (2, 19, 333)]
    for i, (b, d, L) in enumerate(shapes):
        wl = base.with_(batch=b, dim=d, seqlen=L, seed=500 + i)
        inp = wlm.make_inputs(wl, random_A=True, random_D=True)
        t = upload(inp)
        say("case noalloc call %d %s %s" % (i, wl.dtype, (b, d, L)))
        y_na = torch.empty(b, d, L, dtype=torch_dtype(wl), device="cuda")
        y_ws = torch.empty_like(y_na)
        call_noalloc(wl, t, y_na)
        call_with_workspace(wl, t, y_ws)
        torch.cuda.synchronize()
        got, ref_ws = host64(y_na), host64(y_ws)
        bad = np.abs(got - ref_ws) > TOL[wl.dtype] * (1.0 + np.abs(ref_ws))
        assert not bad.any(), "noalloc differs from vim_scan_bidir at %d elements" % int(bad.sum())
        assert torch.equal(y_na, y_ws)     # same kernels on the same inputs
        assert_close(got, oracle.run_inputs(inp), wl.dtype, "noalloc vs oracle")


def test_noalloc_at_the_headline_size():
    """Vim-S 1024^2 (batch 8, 4,097 tokens, 768 channels: 25.2 M elements)
    fits the static buffer; the output equals the workspace entry point's."""
    wl = wlm.WORKLOADS[2]
    inp = wlm.make_inputs(wl)
    t = upload(inp)
    say("case noalloc headline")
    y_na = torch.empty(wl.batch, wl.dim, wl.seqlen, dtype=torch.bfloat16, device="cuda")
    y_ws = torch.empty_like(y_na)
    call_noalloc(wl, t, y_na)
    call_with_workspace(wl, t, y_ws)
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ws)
