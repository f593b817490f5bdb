"""Pins of the oracle's Vim front end and of the per-direction-u scan it
feeds. The guide's BidirectionalVisionMambaBlock ("1. PyTorch Implementation
of the Bidirectional Vision Mamba Block") smooths each branch with a
depthwise Conv1d (kernel 3, padding 1, bias) followed by SiLU, the backward
branch on the flipped sequence. Here PyTorch's own conv1d and silu (CPU,
float64) compute that front end independently, and the unrolled closed form
computes the scan; plausible mistakes planted in a copy of the oracle must
fail these pins."""
import shutil

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from test_oracle_pins import brute_direction, rand_inputs


def torch_front_end(x, w, b):
    """[2, batch, dim, L]: silu(conv_f(x)) and, in token order, the flipped
    branch silu(conv_b(flip(x))) flipped back."""
    xt = torch.from_numpy(np.asarray(x, np.float64))
    dim = x.shape[1]
    out = []
    for k in range(2):
        inp = xt if k == 0 else torch.flip(xt, dims=[2])
        c = torch.nn.functional.conv1d(inp, torch.from_numpy(np.asarray(w[k], np.float64))[:, None, :],
                                       None if b is None else torch.from_numpy(np.asarray(b[k], np.float64)),
                                       padding=1, groups=dim)
        s = torch.nn.functional.silu(c)
        out.append((s if k == 0 else torch.flip(s, dims=[2])).numpy())
    return np.stack(out)


def brute_vim_per_dir_u(uk, dl, z, B, C, A, D, bias):
    """The unrolled closed form with u_k per direction (forward, backward)."""
    _, b_, d_, L = uk.shape
    fwd = np.arange(L)
    orders = [fwd, fwd[::-1].copy()]
    y = np.zeros((b_, d_, L))
    for b in range(b_):
        for d in range(d_):
            tot = np.zeros(L)
            for k, od in enumerate(orders):
                tot += brute_direction(uk[k, b, d], dl[b, d], B[b][:, od], C[b][:, od],
                                       A[k, d], D[k, d], bias[k, d], od)
            if z is not None:
                tot = tot * z[b, d] * scipy.special.expit(z[b, d])
            y[b, d] = tot
    return y


def conv_inputs(rng, batch=2, dim=3, N=4, L=9):
    x, dl, z, B, C, A, D, bias = rand_inputs(rng, batch, dim, N, L, ndir=2)
    w = rng.standard_normal((2, dim, 3))
    cb = rng.standard_normal((2, dim))
    return x, w, cb, dl, z, B, C, A, D, bias


def test_per_direction_u_scan_matches_closed_form(oracle_lib):
    rng = np.random.default_rng(31)
    x, w, cb, dl, z, B, C, A, D, bias = conv_inputs(rng)
    uk = rng.standard_normal((2,) + x.shape)
    got = oracle.scan(uk, dl, z, B, C, A, D, bias, orders=(0, 1), bc_per_direction=False,
                      u_per_direction=True)
    np.testing.assert_allclose(got, brute_vim_per_dir_u(uk, dl, z, B, C, A, D, bias),
                               rtol=1e-11, atol=1e-11)


def test_same_u_in_both_directions_equals_shared_u(oracle_lib):
    rng = np.random.default_rng(32)
    x, w, cb, dl, z, B, C, A, D, bias = conv_inputs(rng)
    got = oracle.scan(np.stack([x, x]), dl, z, B, C, A, D, bias, orders=(0, 1),
                      bc_per_direction=False, u_per_direction=True)
    np.testing.assert_array_equal(got, oracle.vim_bidir(x, dl, z, B, C, A, D, bias))


@pytest.mark.parametrize("with_bias", [True, False])
def test_front_end_matches_torch_conv1d(oracle_lib, with_bias):
    rng = np.random.default_rng(33 + with_bias)
    x, w, cb, dl, z, B, C, A, D, bias = conv_inputs(rng)
    cb = cb if with_bias else None
    got = oracle.vim_conv(x, w, cb, dl, z, B, C, A, D, bias)
    uk = torch_front_end(x, w, cb)
    np.testing.assert_allclose(got, brute_vim_per_dir_u(uk, dl, z, B, C, A, D, bias),
                               rtol=1e-10, atol=1e-11)


def test_identity_kernel_is_silu_of_x(oracle_lib):
    """Taps (0, 1, 0) and no bias leave u = silu(x) in both branches."""
    rng = np.random.default_rng(35)
    x, w, cb, dl, z, B, C, A, D, bias = conv_inputs(rng, L=12)
    w[:] = [0.0, 1.0, 0.0]
    got = oracle.vim_conv(x, w, None, dl, z, B, C, A, D, bias)
    ref = oracle.vim_bidir(x * scipy.special.expit(x), dl, z, B, C, A, D, bias)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_backward_branch_sees_the_flipped_neighbours(oracle_lib):
    """A kernel that reads only its left neighbour (taps 1, 0, 0) reads token
    p-1 in the forward branch and token p+1 in the flipped branch (its left
    neighbour in flipped order), with zeros past either end."""
    rng = np.random.default_rng(36)
    x, w, cb, dl, z, B, C, A, D, bias = conv_inputs(rng, batch=1, dim=2, L=10)
    w[:] = [1.0, 0.0, 0.0]
    left = np.concatenate([np.zeros(x.shape[:2] + (1,)), x[..., :-1]], axis=-1)
    right = np.concatenate([x[..., 1:], np.zeros(x.shape[:2] + (1,))], axis=-1)
    s = lambda v: v * scipy.special.expit(v)
    uk = np.stack([s(left), s(right)])
    got = oracle.vim_conv(x, w, None, dl, z, B, C, A, D, bias)
    np.testing.assert_allclose(got, brute_vim_per_dir_u(uk, dl, z, B, C, A, D, bias),
                               rtol=1e-10, atol=1e-11)


# ---- the pins must be able to fail
CONV_MUTATIONS = {
    "taps_swapped": ("w[0] * left + w[1] * in[t] + w[2] * right",
                     "w[2] * left + w[1] * in[t] + w[0] * right"),
    "bias_dropped": ("out[t] = bias + w[0] * left", "out[t] = 0.0 * bias + w[0] * left"),
    "padding_wraps": ("const double left = t > 0 ? in[t - 1] : 0.0;",
                      "const double left = t > 0 ? in[t - 1] : in[L - 1];"),
    "backward_not_flipped": ("rev[t] = xr[L - 1 - t];", "rev[t] = xr[t];"),
    "backward_not_flipped_back": ("u[(rows + r) * L + (L - 1 - t)] = silu(c[t]);",
                                  "u[(rows + r) * L + t] = silu(c[t]);"),
    "sigmoid_not_silu": ("static double silu(double v) { return v / (1.0 + exp(-v)); }",
                         "static double silu(double v) { return 1.0 / (1.0 + exp(-v)); }"),
    "u_shared_not_per_direction": ("((J->per_direction & PER_DIR_U) ? k * copy : 0)", "0"),
    "backward_uses_forward_taps": ("conv_w + ((long)dim + d) * 3", "conv_w + d * 3"),
}


def conv_battery(lib):
    rng = np.random.default_rng(4321)
    x, w, cb, dl, z, B, C, A, D, bias = conv_inputs(rng, batch=1, dim=2, N=3, L=7)
    try:
        got = oracle.vim_conv(x, w, cb, dl, z, B, C, A, D, bias, lib=lib, nthreads=2)
    except ValueError:
        return ["front_end"]
    ref = brute_vim_per_dir_u(torch_front_end(x, w, cb), dl, z, B, C, A, D, bias)
    return [] if np.allclose(got, ref, rtol=1e-10, atol=1e-10) else ["front_end"]


def _build(tmp_path, name, text):
    src = tmp_path / (name + ".c")
    src.write_text(text)
    out = tmp_path / ("lib" + name + ".so")
    oracle.build(force=True, src=str(src), out=str(out))
    return oracle.load(str(out))


@pytest.fixture(scope="module")
def source():
    with open(oracle._SRC) as f:
        return f.read()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_unmodified_source_passes_conv_battery(tmp_path, source):
    assert conv_battery(_build(tmp_path, "orig", source)) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(CONV_MUTATIONS))
def test_conv_mutant_is_caught(tmp_path, source, name):
    old, new = CONV_MUTATIONS[name]
    assert source.count(old) == 1, "mutation anchor missing: %s" % name
    assert conv_battery(_build(tmp_path, name, source.replace(old, new))), \
        "planted mistake %r passed the front-end pins" % name
