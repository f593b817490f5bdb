"""GPU parity of the linear maps around the scan (vim_x_proj, vim_dt_proj,
vim_out_proj) against the fp64 oracle, element by element, through the C
ABI.

Bound, from the arithmetic: inputs are bf16-exact, products are exact in
fp32 and the matrix cores accumulate in fp32, so |g - ref| <= 2^-8 |ref|
(the final round to bf16, half an ulp, with margin) + K 2^-23 sum_k |W| |X|
(fp32 accumulation over K terms in any order). The fp32 dt of x_proj has
no final rounding, so only the second term applies."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_finite, dev, host64, say
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu


def bf16(a):
    return wlm.round_bf16(np.asarray(a, np.float32))


def check(got, ref, absdot, K, what, rounded=True):
    assert_finite(got, ref, what)
    tol = K * 2.0 ** -23 * absdot + (2.0 ** -8 * np.abs(ref) if rounded else 0.0)
    bad = np.abs(got - ref) > tol
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d beyond the bound; first at %s: got %r ref %r tol %r" % (
            what, int(bad.sum()), bad.size, i, got[i], ref[i], tol[i]))
    say("  %s max |err| / |ref| %.3g" % (what, float(np.max(np.abs(got - ref) / (1e-30 + np.abs(ref))))))


def operands(rng, batch, K, M, L):
    x = bf16(rng.standard_normal((batch, K, L)))
    W = bf16(rng.standard_normal((M, K)) / np.sqrt(K))
    return x, W


@pytest.mark.parametrize("shape", [(2, 24, 16, 37), (1, 100, 16, 130), (3, 8, 8, 65),
                                   (1, 64, 4, 1), (2, 200, 16, 300), (1, 136, 8, 70)])
def test_x_proj(shape):
    import vision_mamba_selective_amd as vms
    batch, dim, N, L = shape
    rng = np.random.default_rng(sum(shape) + 5)
    u, W = operands(rng, batch, dim, 2 * N + 1, L)
    say("case x_proj %s" % (shape,))
    B, C, dt = vms.vim_x_proj(dev(u, torch.bfloat16), dev(W, torch.bfloat16), N)
    rB, rC, rdt = oracle.x_proj(W, u, N)
    absdot = oracle.linear(np.abs(W), np.abs(u))
    check(host64(B), rB, absdot[:, :N], dim, "B")
    check(host64(C), rC, absdot[:, N:2 * N], dim, "C")
    check(host64(dt), rdt, absdot[:, 2 * N], dim, "dt", rounded=False)


@pytest.mark.parametrize("shape", [(2, 24, 37), (1, 130, 1), (3, 8, 300)])
def test_dt_proj(shape):
    import vision_mamba_selective_amd as vms
    batch, dim, L = shape
    rng = np.random.default_rng(sum(shape) + 6)
    dt = rng.standard_normal((batch, L)).astype(np.float32)
    w = rng.standard_normal(dim).astype(np.float32)
    say("case dt_proj %s" % (shape,))
    got = host64(vms.vim_dt_proj(dev(dt, torch.float32), dev(w, torch.float32)))
    ref = oracle.dt_proj(dt, w)
    check(got, ref, np.zeros_like(ref), 1, "delta")


@pytest.mark.parametrize("bias,res", [(True, True), (False, False), (True, False), (False, True)])
@pytest.mark.parametrize("shape", [(2, 64, 48, 37), (1, 100, 130, 200), (2, 256, 256, 300),
                                   (1, 8, 3, 1), (2, 64, 160, 72), (1, 72, 64, 71),
                                   (1, 64, 160, 1031), (2, 96, 136, 1100), (1, 200, 96, 1100),
                                   (1, 136, 130, 1030)])
def test_out_proj(shape, bias, res):
    import vision_mamba_selective_amd as vms
    batch, din, dout, L = shape
    rng = np.random.default_rng(sum(shape) + 7 + 2 * bias + res)
    y, W = operands(rng, batch, din, dout, L)
    b = rng.standard_normal(dout).astype(np.float32) if bias else None
    r = bf16(rng.standard_normal((batch, dout, L))) if res else None
    say("case out_proj %s bias=%s residual=%s" % (shape, bias, res))
    got = host64(vms.vim_out_proj(dev(y, torch.bfloat16), dev(W, torch.bfloat16),
                                  dev(b, torch.float32), dev(r, torch.bfloat16)))
    check(got, oracle.linear(W, y, b, r), oracle.linear(np.abs(W), np.abs(y)), din, "out")


def test_out_proj_in_place_residual():
    import vision_mamba_selective_amd as vms
    rng = np.random.default_rng(8)
    y, W = operands(rng, 2, 96, 96, 77)
    r = bf16(rng.standard_normal((2, 96, 77)))
    rt = dev(r, torch.bfloat16)
    say("case out_proj in place")
    o = vms.vim_out_proj(dev(y, torch.bfloat16), dev(W, torch.bfloat16), None, rt, out=rt)
    assert o.data_ptr() == rt.data_ptr()
    check(host64(rt), oracle.linear(W, y, None, r), oracle.linear(np.abs(W), np.abs(y)), 96, "out")


def sample_tokens(L, tile=64, seed=7):
    """One seeded column inside every 64-token tile, plus the tiles' edges
    around 128 and the last token: every token tile of the output is
    checked."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, L, tile)
    inner = starts + rng.integers(0, tile, starts.size)
    return np.unique(np.concatenate([np.minimum(inner, L - 1), [0, 127, 128, L - 1]]))


def test_projections_workload_full_size():
    """The Vim-S 1024x1024 block's projections at full size (batch 8, 768
    channels, 4,097 tokens); the oracle recomputes one token column in every
    64-token tile, for every batch row and output channel (every output
    column depends on its own input column only)."""
    import vision_mamba_selective_amd as vms
    wl = wlm.WORKLOADS[2]
    rng = np.random.default_rng(2025)
    u, Wo = operands(rng, wl.batch, wl.dim, wl.dim, wl.seqlen)
    Wx = bf16(rng.standard_normal((2 * wl.dstate + 1, wl.dim)) / np.sqrt(wl.dim))
    bo = rng.standard_normal(wl.dim).astype(np.float32)
    ts = sample_tokens(wl.seqlen)
    us = u[:, :, ts]
    say("case projections full size %s" % wl.name)
    ut = dev(u, torch.bfloat16)
    B, C, dt = vms.vim_x_proj(ut, dev(Wx, torch.bfloat16), wl.dstate)
    rB, rC, rdt = oracle.x_proj(Wx, us, wl.dstate)
    ax = oracle.linear(np.abs(Wx), np.abs(us))
    N = wl.dstate
    check(host64(B)[:, :, ts], rB, ax[:, :N], wl.dim, "B")
    check(host64(C)[:, :, ts], rC, ax[:, N:2 * N], wl.dim, "C")
    check(host64(dt)[:, ts], rdt, ax[:, 2 * N], wl.dim, "dt", rounded=False)
    o = vms.vim_out_proj(ut, dev(Wo, torch.bfloat16), dev(bo, torch.float32), ut.clone())
    ref = oracle.linear(Wo, us, bo, us)
    check(host64(o)[:, :, ts], ref, oracle.linear(np.abs(Wo), np.abs(us)), wl.dim, "out")
