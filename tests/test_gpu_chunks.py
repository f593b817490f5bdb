"""GPU parity of the chunked Vim scan (vim_scan_bidir_chunked): every chunk
count gives the oracle's result, and the chunk counts agree with each other
to fp32 rounding (chunk-count invariance), on ragged lengths, both dtypes,
with and without gate and softplus, and at the Vim-B 2048^2 shape that the
library chunks on its own."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (STRICT, assert_close, host64, say, stable_without_softplus, strict_bound,
                      strict_err, upload)
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu

VIM_F32 = wlm.WORKLOADS[0]
VIM_BF16 = wlm.WORKLOADS[1]


def run(inp, chunks, delta_softplus=True, t=None):
    import vision_mamba_selective_amd as vms
    t = t or upload(inp)
    return vms.vim_scan_bidir_chunked(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"],
                                      t["Dskip"], t["dt_bias"], chunks=chunks,
                                      delta_softplus=delta_softplus)


# batch, dim, L: several tiles and a ragged last one, a single tile, two
# tiles with a one-token tail, channels that leave workgroup rows idle
SHAPES = [(2, 13, 1000), (1, 8, 33), (3, 17, 257), (1, 9, 4097), (2, 5, 96)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_every_chunk_count_matches_the_oracle(shape, base):
    b, d, L = shape
    wl = base.with_(batch=b, dim=d, seqlen=L, seed=3000 + L + d)
    inp = wlm.make_inputs(wl, random_A=True, random_D=True)
    ref = oracle.run_inputs(inp)
    t = upload(inp)
    ntile = (L + 31) // 32
    for k in (1, 2, 3, 4, 8, 64):
        say("case chunks=%d %s %s" % (k, wl.dtype, shape))
        y = host64(run(inp, k, t=t))
        err = assert_close(y, ref, wl.dtype, "chunks %d (of at most %d)" % (k, ntile))
        say("  max rel err %.3g" % err)


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_chunk_count_invariance_strict(base):
    """D = 0 and no gate, random A: every chunk count agrees with the oracle
    to the strict scan-only bound, so a carry that is wrong by a little (a
    dropped decay, a wrong piece boundary) cannot hide."""
    wl = base.with_(batch=2, dim=24, seqlen=2000, gate=False, seed=77)
    inp = wlm.make_inputs(wl, random_A=True)
    inp.D[:] = 0.0
    ref = oracle.run_inputs(inp)
    t = upload(inp)
    for k in (1, 2, 4, 8, 16):
        y = host64(run(inp, k, t=t))
        err, rms = strict_err(y, ref, wl.dtype)
        say("case strict chunks=%d %s: %.3g (rms %.3g)" % (k, wl.dtype, err, rms))
        assert err <= strict_bound(wl.dtype, wl.seqlen)


@pytest.mark.parametrize("base", [VIM_F32, VIM_BF16], ids=["f32", "bf16"])
def test_chunks_without_gate_and_softplus(base):
    wl = base.with_(batch=2, dim=11, seqlen=700, gate=False, seed=91)
    inp = stable_without_softplus(wlm.make_inputs(wl, random_D=True))
    ref = oracle.vim_bidir(inp.u, inp.delta, None, inp.B, inp.C, inp.A, inp.D, inp.dt_bias,
                           delta_softplus=False)
    for k in (2, 3, 5):
        say("case chunks=%d softplus off %s" % (k, wl.dtype))
        assert_close(host64(run(inp, k, delta_softplus=False)), ref, wl.dtype, "softplus off")


def test_delta_zero_is_exact_with_chunks():
    """delta = 0 (softplus off, no bias): every carry is zero and
    y = D_f u + D_b u = 2u exactly, whatever the chunk count."""
    import vision_mamba_selective_amd as vms
    wl = VIM_BF16.with_(batch=2, dim=9, seqlen=500, gate=False)
    inp = wlm.make_inputs(wl)
    inp.delta[:] = 0.0
    t = upload(inp)
    for k in (2, 4, 7):
        y = vms.vim_scan_bidir_chunked(t["u"], t["delta"], None, t["B"], t["C"], t["A"],
                                       t["Dskip"], None, chunks=k, delta_softplus=False)
        assert torch.equal(y, 2 * t["u"])


def test_vim_b_2048_chunk_counts():
    """The Vim-B 2048^2 workload (batch 2, 16,385 tokens, 1,536 channels),
    which vim_scan_bidir chunks on its own: one, two and four chunks against
    the oracle, every element."""
    wl = wlm.WORKLOADS[4]
    inp = wlm.make_inputs(wl)
    ref = oracle.run_inputs(inp)
    t = upload(inp)
    for k in (1, 2, 4):
        say("case vim_b_2048 chunks=%d" % k)
        y = host64(run(inp, k, t=t))
        err = assert_close(y, ref, wl.dtype, "vim_b_2048 chunks %d" % k)
        say("  max rel err %.3g" % err)


def test_chunked_repeatable_and_in_bounds():
    """Two runs give identical bits; nothing outside y is written."""
    wl = VIM_BF16.with_(batch=3, dim=21, seqlen=611)
    inp = wlm.make_inputs(wl)
    t = upload(inp)
    n = wl.batch * wl.dim * wl.seqlen
    guard = 4096
    canary = torch.full((n + 2 * guard,), 7.25, dtype=torch.bfloat16, device="cuda")
    out = canary[guard:guard + n].view(wl.batch, wl.dim, wl.seqlen)
    import vision_mamba_selective_amd as vms
    say("case chunked repeat/canary")
    y1 = vms.vim_scan_bidir_chunked(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"],
                                    t["Dskip"], t["dt_bias"], chunks=3, out=out).clone()
    y2 = run(inp, 3, t=t)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.all(canary[:guard] == 7.25) and torch.all(canary[guard + n:] == 7.25)
