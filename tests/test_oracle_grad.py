"""Pins of the oracle's gradient of the Vim scan (reverse mode through the
sequential definition). Two independent references:
  * PyTorch autograd through a separate float64 PyTorch implementation of
    the forward definition (a step loop vectorised over batch, channel and
    state), and
  * central finite differences of the (already pinned) forward oracle along
    random directions.
Plausible mistakes planted in a copy of the oracle must fail them."""
import shutil

import numpy as np
import pytest
import torch

import oracle
from test_oracle_pins import rand_inputs


def torch_forward(u, dl, z, B, C, A, D, bias, softplus=True):
    """Vim forward in float64 PyTorch: per direction a loop over steps,
    h = exp(delta A) h + delta B_t u_t, y_t = C_t h + D u_t; merged and gated."""
    L = u.shape[-1]
    out = torch.zeros_like(u)
    for k in range(2):
        x = dl + bias[k][None, :, None]
        delta = torch.nn.functional.softplus(x) if softplus else x
        h = torch.zeros(u.shape[0], u.shape[1], A.shape[-1], dtype=u.dtype)
        ys = [None] * L
        steps = range(L) if k == 0 else range(L - 1, -1, -1)
        for p in steps:
            dp = delta[:, :, p, None]
            h = torch.exp(dp * A[k][None]) * h + dp * B[:, None, :, p] * u[:, :, p, None]
            ys[p] = (C[:, None, :, p] * h).sum(-1) + D[k][None] * u[:, :, p]
        out = out + torch.stack(ys, dim=-1)
    if z is not None:
        out = out * torch.nn.functional.silu(z)
    return out


def autograd_reference(args, g, softplus=True):
    u, dl, z, B, C, A, D, bias = args
    t = [None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True)
         for a in (u, dl, z, B, C, A, D, bias)]
    y = torch_forward(*t, softplus=softplus)
    (y * torch.tensor(g)).sum().backward()
    names = ("du", "ddelta", "dz", "dB", "dC", "dA", "dD", "ddt_bias")
    return {n: (np.zeros_like(a) if v is None else v.grad.numpy())
            for n, v, a in zip(names, t, (u, dl, u, B, C, A, D, bias))}


def check(got, ref, rtol=1e-9, atol=1e-10):
    for k in ref:
        np.testing.assert_allclose(got[k], ref[k], rtol=rtol, atol=atol, err_msg=k)


@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("softplus", [True, False])
def test_grad_matches_autograd(oracle_lib, gate, softplus):
    rng = np.random.default_rng(50 + 2 * gate + softplus)
    args = rand_inputs(rng, batch=2, dim=3, N=4, L=11, ndir=2, gate=gate)
    if not softplus:
        args = args[:1] + (np.abs(args[1]) * 0.3,) + args[2:]
    g = rng.standard_normal(args[0].shape)
    got = oracle.vim_bidir_grad(*args, g, delta_softplus=softplus)
    check(got, autograd_reference(args, g, softplus))


def test_grad_matches_finite_differences(oracle_lib):
    """<grad, v> against (f(x + eps v) - f(x - eps v)) / (2 eps) for f = <g, y>,
    with the forward oracle, for each input in turn."""
    rng = np.random.default_rng(60)
    args = list(rand_inputs(rng, batch=1, dim=2, N=3, L=9, ndir=2))
    g = rng.standard_normal(args[0].shape)
    grads = oracle.vim_bidir_grad(*args, g)
    f = lambda a: float(np.sum(g * oracle.vim_bidir(*a)))
    names = ("du", "ddelta", "dz", "dB", "dC", "dA", "dD", "ddt_bias")
    eps = 1e-6
    for i, name in enumerate(names):
        v = rng.standard_normal(args[i].shape)
        plus = list(args)
        minus = list(args)
        plus[i] = args[i] + eps * v
        minus[i] = args[i] - eps * v
        fd = (f(plus) - f(minus)) / (2 * eps)
        an = float(np.sum(grads[name] * v))
        assert abs(fd - an) <= 1e-6 * (1 + abs(an)), (name, fd, an)


def test_zero_upstream_gradient_gives_zero(oracle_lib):
    rng = np.random.default_rng(61)
    args = rand_inputs(rng, batch=1, dim=2, N=3, L=7, ndir=2)
    got = oracle.vim_bidir_grad(*args, np.zeros(args[0].shape))
    for k, v in got.items():
        assert not np.any(v), k


def test_threads_do_not_change_gradients(oracle_lib):
    rng = np.random.default_rng(62)
    args = rand_inputs(rng, batch=3, dim=5, N=4, L=13, ndir=2)
    g = rng.standard_normal(args[0].shape)
    one = oracle.vim_bidir_grad(*args, g, nthreads=1)
    many = oracle.vim_bidir_grad(*args, g, nthreads=7)
    check(many, one, rtol=1e-13, atol=1e-14)


# ---- the pins must be able to fail
GRAD_MUTATIONS = {
    "adjoint_without_decay": ("lam[n] = gs[p] * Cb[n * L + p] + e_next * lam[n];",
                              "lam[n] = gs[p] * Cb[n * L + p] + lam[n];"),
    "decay_of_this_step": ("exp(next_delta * A[n])", "exp(delta * A[n])"),
    "dB_without_delta": ("dBb[n * L + p] += lam[n] * delta * u[p];",
                         "dBb[n * L + p] += lam[n] * u[p];"),
    "dC_with_adjoint": ("dCb[n * L + p] += gs[p] * h[t * N + n];",
                        "dCb[n * L + p] += lam[n] * h[t * N + n];"),
    "ddelta_missing_input_term": ("(hprev * e * A[n] + Bb[n * L + p] * u[p])", "(hprev * e * A[n])"),
    "dA_current_state": ("dA[n] += lam[n] * hprev * e * delta;",
                         "dA[n] += lam[n] * h[t * N + n] * e * delta;"),
    "softplus_derivative_wrong": ("ddelta * (J->delta_softplus ? sigmoid(x) : 1.0)",
                                  "ddelta * (J->delta_softplus ? 1.0 : 1.0)"),
    "gate_derivative_is_sigmoid": ("dz[p] = g[p] * s[p] * sg * (1.0 + zz * (1.0 - sg));",
                                   "dz[p] = g[p] * s[p] * sg;"),
    "skip_gradient_dropped": ("du[p] += gs[p] * Dk + dupart;", "du[p] += dupart;"),
}


def grad_battery(lib):
    rng = np.random.default_rng(6543)
    args = rand_inputs(rng, batch=1, dim=2, N=3, L=6, ndir=2)
    g = rng.standard_normal(args[0].shape)
    try:
        got = oracle.vim_bidir_grad(*args, g, lib=lib, nthreads=2)
    except ValueError:
        return ["grad"]
    ref = autograd_reference(args, g)
    bad = [k for k in ref if not np.allclose(got[k], ref[k], rtol=1e-9, atol=1e-10)]
    return bad


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
def test_unmodified_source_passes_grad_battery(tmp_path, source):
    assert grad_battery(_build(tmp_path, "orig", source)) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(GRAD_MUTATIONS))
def test_grad_mutant_is_caught(tmp_path, source, name):
    old, new = GRAD_MUTATIONS[name]
    assert source.count(old) == 1, "mutation anchor missing: %s" % name
    assert grad_battery(_build(tmp_path, name, source.replace(old, new))), \
        "planted mistake %r passed the gradient pins" % name
