"""GPU parity of the VMamba four-direction cross-scan against the fp64 oracle,
element by element, through the C ABI. Grids are mostly non-square (H != W),
so a swapped row/column index cannot pass."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (STRICT, assert_close, host64, run_gpu, say, stable_without_softplus, strict_bound,
                      strict_err, upload)
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu

X4_F32 = wlm.WORKLOADS[3]
X4_BF16 = X4_F32.with_(dtype=wlm.BF16)


def make(base, batch, dim, H, W, dstate=16, gate=False, seed=0, **kw):
    wl = base.with_(batch=batch, dim=dim, H=H, W=W, seqlen=H * W, dstate=dstate, gate=gate,
                    seed=seed)
    return wlm.make_inputs(wl, **kw)


def check(inp, what, **kw):
    say("case %s %s" % (what, inp.wl))
    y = host64(run_gpu(inp, **kw))
    ref = oracle.run_inputs(inp)
    err = assert_close(y, ref, inp.wl.dtype, what)
    say("  max rel err %.3g" % err)
    return y, ref


# batch, dim, H, W, dstate: several 16-token blocks with ragged tails, grids
# of one row or one column, and blocks that wrap several columns (H < 16)
SMALL = [
    (1, 1, 1, 1, 16),
    (1, 3, 5, 7, 16),
    (2, 5, 7, 5, 16),
    (1, 4, 1, 13, 16),
    (1, 4, 13, 1, 16),
    (2, 6, 16, 16, 16),
    (1, 9, 9, 23, 8),
    (1, 5, 3, 37, 16),
    (2, 3, 17, 4, 1),
    (1, 7, 40, 33, 12),
]


@pytest.mark.parametrize("gate", [False, True], ids=["sum", "gated"])
@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("base", [X4_F32, X4_BF16], ids=["f32", "bf16"])
def test_cross4_small(shape, base, gate):
    b, d, H, W, N = shape
    inp = make(base, b, d, H, W, N, gate=gate, seed=sum(shape) * 11 + gate,
               random_A=True, random_D=True)
    check(inp, "small%s gate=%s" % (shape, gate))


@pytest.mark.parametrize("base", [X4_F32, X4_BF16], ids=["f32", "bf16"])
def test_cross4_softplus_off(base):
    inp = make(base, 2, 6, 11, 9, seed=5, random_D=True)
    stable_without_softplus(inp)
    say("case cross4 softplus off")
    y = host64(run_gpu(inp, delta_softplus=False))
    ref = oracle.cross4(inp.u, inp.delta, None, inp.B, inp.C, inp.A, inp.D, inp.dt_bias, 11, 9,
                        delta_softplus=False)
    assert_close(y, ref, base.dtype, "softplus off")


@pytest.mark.parametrize("base", [X4_F32, X4_BF16], ids=["f32", "bf16"])
def test_cross4_scan_only_strict(base):
    """D = 0 and no gate: the output is the four scan terms alone."""
    inp = make(base, 2, 12, 24, 19, seed=9, random_A=True)
    inp.D[:] = 0.0
    say("case cross4 scan-only strict %s" % base.dtype)
    y = host64(run_gpu(inp))
    ref = oracle.run_inputs(inp)
    err, rms = strict_err(y, ref, base.dtype)
    say("  max (|dy| - output rounding) / rms = %.3g (rms %.3g)" % (err, rms))
    assert err <= STRICT[base.dtype]


@pytest.mark.parametrize("base", [X4_F32, X4_BF16], ids=["f32", "bf16"])
def test_cross4_delta_zero_is_four_u(base):
    """delta = 0 (softplus off, no bias) keeps every state at 0, so with
    D_k = 1 the merge of the four directions returns exactly 4u."""
    import vision_mamba_selective_amd as vms
    inp = make(base, 2, 5, 6, 11, seed=3)
    inp.delta[:] = 0.0
    t = upload(inp)
    say("case cross4 delta zero")
    y = vms.vmamba_cross_scan4(t["u"], t["delta"], None, t["B"], t["C"], t["A"], 6, 11,
                               t["Dskip"], None, delta_softplus=False)
    assert torch.equal(y, 4 * t["u"])


def visit_order(k, H, W):
    """Token visited at each scan step by direction k, from numpy transposes
    of the row-major grid."""
    row = np.arange(H * W)
    col = row.reshape(H, W).T.reshape(-1)
    return [row, row[::-1], col, col[::-1]][k]


@pytest.mark.parametrize("k", [0, 1, 2, 3])
@pytest.mark.parametrize("base", [X4_F32, X4_BF16], ids=["f32", "bf16"])
def test_cross4_single_direction(k, base):
    """C_j = 0 and D_j = 0 for every direction j != k: the cross-scan reduces
    to the one-direction scan of direction k's traversal of the grid."""
    H, W = 7, 12
    inp = make(base, 2, 6, H, W, seed=20 + k, random_A=True, random_D=True)
    for j in range(4):
        if j != k:
            inp.C[:, j] = 0.0
            inp.D[j] = 0.0
    say("case cross4 single direction %d" % k)
    y = host64(run_gpu(inp))
    order = visit_order(k, H, W)
    yk = oracle.s6_1d(inp.u[..., order], inp.delta[..., order], None, inp.B[:, k], inp.C[:, k],
                      inp.A[k], inp.D[k], inp.dt_bias[k])
    ref = np.empty_like(yk)
    ref[..., order] = yk
    assert_close(y, ref, base.dtype, "direction %d" % k)


def test_cross4_repeatable_and_in_bounds():
    """Two runs give identical bits whatever the workspace held; nothing
    outside y is written."""
    import vision_mamba_selective_amd as vms
    inp = make(X4_BF16, 3, 7, 13, 9, gate=True, seed=31)
    wl = inp.wl
    t = upload(inp)
    n = wl.batch * wl.dim * wl.seqlen
    guard = 4096
    canary = torch.full((n + 2 * guard,), 7.25, dtype=torch.bfloat16, device="cuda")
    out = canary[guard:guard + n].view(wl.batch, wl.dim, wl.seqlen)
    need = vms.workspace_bytes(1, wl.batch, wl.dim, wl.seqlen, torch.bfloat16)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    say("case cross4 repeat/canary")
    y1 = vms.vmamba_cross_scan4(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], wl.H, wl.W,
                                t["Dskip"], t["dt_bias"], out=out, workspace=ws).clone()
    y2 = run_gpu(inp, t)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.all(canary[:guard] == 7.25) and torch.all(canary[guard + n:] == 7.25)


# ---- the 64 x 64 grid workload at full size, in the launch configuration the
# benchmark times; every element of y is compared with the oracle.
@pytest.mark.parametrize("base", [X4_F32, X4_BF16], ids=["f32", "bf16"])
def test_cross4_workload_full_size(base):
    wl = base
    say("case workload %s %s" % (wl.name, wl.dtype))
    inp = wlm.make_inputs(wl)
    y = host64(run_gpu(inp))
    ref = oracle.run_inputs(inp)
    err = assert_close(y, ref, wl.dtype, wl.name)
    say("  %s max rel err %.3g over all %d outputs" % (wl.name, err, y.size))


def test_cross4_scan_only_strict_full_size():
    """D = 0, no gate, random A on the full 64 x 64 grid (fp32): the four
    orders' carries over 4,096 steps each, with nothing to hide under."""
    wl = X4_F32.with_(gate=False)
    say("case cross4 scan-only strict full size")
    inp = wlm.make_inputs(wl, random_A=True)
    inp.D[:] = 0.0
    y = host64(run_gpu(inp))
    ref = oracle.run_inputs(inp)
    err, rms = strict_err(y, ref, wl.dtype)
    say("  max |dy| / rms = %.3g (rms %.3g)" % (err, rms))
    assert err <= strict_bound(wl.dtype, wl.seqlen)


# Grids whose u and delta fit the LDS budget (8 KB for a workgroup's 4
# channels: fp32 up to 256 tokens, bf16 up to 512) are staged there in
# column-major order; larger ones read transposed copies from the workspace.
# Both sides of the limit, with H != W and channel counts that leave idle
# channels in the last workgroup.
GRID_EDGE = [
    # dtype base, H, W, dim
    ("f32", 16, 16, 5),      # 256 tokens: the largest fp32 grid in LDS
    ("f32", 11, 24, 6),      # 264: transposed copies
    ("f32", 7, 7, 7),        # a VMamba stage grid
    ("bf16", 16, 32, 5),     # 512 tokens: the largest bf16 grid in LDS
    ("bf16", 19, 27, 3),     # 513: transposed copies
    ("bf16", 14, 14, 9),     # a VMamba stage grid
]


@pytest.mark.parametrize("case", GRID_EDGE, ids=["%s-%dx%d" % c[:3] for c in GRID_EDGE])
def test_cross4_either_side_of_the_lds_grid_limit(case):
    import vision_mamba_selective_amd as vms
    name, H, W, d = case
    base = X4_F32 if name == "f32" else X4_BF16
    inp = make(base, 2, d, H, W, gate=True, seed=H * W + d, random_A=True, random_D=True)
    tdt = torch.float32 if name == "f32" else torch.bfloat16
    es = 4 if name == "f32" else 2
    in_lds = 2 * 4 * H * W * es <= 8 * 1024
    e = 2 * d * H * W
    bufs = (1 if name == "f32" else 2) * e * 4
    assert vms.workspace_bytes(1, 2, d, H * W, tdt) == bufs + (0 if in_lds else 2 * e * es)
    check(inp, "grid edge %s %dx%d (%s)" % (name, H, W, "LDS" if in_lds else "copies"))
