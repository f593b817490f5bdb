"""Pins of the oracle's linear maps around the scan (x_proj, dt_proj,
out_proj). The guide's "1. PyTorch Implementation of the Bidirectional Vision
Mamba Block" builds them from nn.Linear on token-major (batch, L, features)
tensors; here PyTorch's own linear (CPU, float64) on that layout is the
reference for the oracle's channel-major loops, and the guide's
SimpleSelectiveSSM forward, written in PyTorch, checks how x_proj, dt_proj
and the scan compose. Planted mistakes in a copy of the oracle must fail."""
import shutil

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def tm(a):
    """channel-major [batch, feat, L] -> token-major [batch, L, feat] tensor"""
    return torch.from_numpy(np.ascontiguousarray(np.swapaxes(a, 1, 2)))


def cm(t):
    """token-major tensor -> channel-major array"""
    return np.swapaxes(t.numpy(), 1, 2)


@pytest.mark.parametrize("with_bias,with_res", [(True, True), (False, False), (True, False)])
def test_linear_matches_torch(oracle_lib, with_bias, with_res):
    rng = np.random.default_rng(91)
    batch, K, M, L = 2, 7, 5, 11
    x = rng.standard_normal((batch, K, L))
    W = rng.standard_normal((M, K))
    b = rng.standard_normal(M) if with_bias else None
    r = rng.standard_normal((batch, M, L)) if with_res else None
    ref = F.linear(tm(x), torch.from_numpy(W), None if b is None else torch.from_numpy(b))
    ref = cm(ref) + (r if r is not None else 0.0)
    np.testing.assert_allclose(oracle.linear(W, x, b, r), ref, rtol=1e-13, atol=1e-13)


def test_x_proj_and_dt_proj_match_the_code_slices(oracle_lib):
    rng = np.random.default_rng(92)
    batch, D, N, L = 2, 6, 4, 9
    u = rng.standard_normal((batch, D, L))
    Wx = rng.standard_normal((2 * N + 1, D))
    wdt = rng.standard_normal(D)
    proj = F.linear(tm(u), torch.from_numpy(Wx))            # (batch, L, 2N + 1)
    B, C, dt = oracle.x_proj(Wx, u, N)
    np.testing.assert_allclose(B, cm(proj[:, :, :N]), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(C, cm(proj[:, :, N:2 * N]), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dt, proj[:, :, 2 * N].numpy(), rtol=1e-13, atol=1e-13)
    widened = F.linear(proj[:, :, 2 * N:], torch.from_numpy(wdt[:, None]))   # Linear(1, D)
    np.testing.assert_allclose(oracle.dt_proj(dt, wdt), cm(widened), rtol=1e-13, atol=1e-13)


def guide_ssm_forward(x, Wx, wdt, bdt, A_log):
    """SimpleSelectiveSSM.forward as the guide writes it, in float64
    PyTorch: x (batch, L, D) -> y (batch, L, D)."""
    N = A_log.shape[1]
    proj = F.linear(x, Wx)
    Bp, Cp, dtp = proj[:, :, :N], proj[:, :, N:2 * N], proj[:, :, 2 * N:]
    delta = F.softplus(F.linear(dtp, wdt[:, None], bdt))
    A = -torch.exp(A_log)
    dA = torch.exp(delta.unsqueeze(-1) * A)
    dB = delta.unsqueeze(-1) * Bp.unsqueeze(2)
    h = torch.zeros(x.shape[0], x.shape[2], N, dtype=x.dtype)
    ys = []
    for t in range(x.shape[1]):
        h = dA[:, t] * h + dB[:, t] * x[:, t, :].unsqueeze(-1)
        ys.append((h * Cp[:, t].unsqueeze(1)).sum(-1))
    return torch.stack(ys, dim=1)


def test_projections_compose_into_the_guide_ssm(oracle_lib):
    """x_proj -> dt_proj (its bias as the scan's dt_bias) -> one-direction
    scan with D = 0 and A = -exp(A_log) reproduces SimpleSelectiveSSM."""
    rng = np.random.default_rng(93)
    batch, D, N, L = 2, 5, 4, 13
    u = rng.standard_normal((batch, D, L))
    Wx = 0.4 * rng.standard_normal((2 * N + 1, D))
    wdt, bdt = rng.standard_normal(D), rng.standard_normal(D)
    A_log = np.log(np.arange(1, N + 1, dtype=np.float64))[None].repeat(D, 0)
    ref = guide_ssm_forward(tm(u), torch.from_numpy(Wx), torch.from_numpy(wdt),
                            torch.from_numpy(bdt), torch.from_numpy(A_log))
    B, C, dt = oracle.x_proj(Wx, u, N)
    delta = oracle.dt_proj(dt, wdt)
    y = oracle.s6_1d(u, delta, None, B, C, -np.exp(A_log), np.zeros(D), bdt)
    np.testing.assert_allclose(y, cm(ref), rtol=1e-11, atol=1e-12)


# ---- the pins must be able to fail
PROJ_MUTATIONS = {
    "weight_transposed": ("W[m * K + k] * in[(b * K + k) * L + t]",
                          "W[k * M + m] * in[(b * K + k) * L + t]"),
    "bias_dropped": ("if (bias) s += bias[m];", "if (bias) s += 0.0;"),
    "residual_dropped": ("if (residual) s += residual[(b * M + m) * L + t];", ""),
    "input_token_shifted": ("in[(b * K + k) * L + t]", "in[(b * K + k) * L + (t + 1) % L]"),
    "dt_weight_of_token": ("w[d] * dt[b * L + t]", "w[t % dim] * dt[b * L + t]"),
}


def proj_battery(lib):
    rng = np.random.default_rng(4323)
    batch, K, M, L = 2, 4, 3, 6
    x = rng.standard_normal((batch, K, L))
    W = rng.standard_normal((M, K))
    b = rng.standard_normal(M)
    r = rng.standard_normal((batch, M, L))
    w = rng.standard_normal(5)
    dt = rng.standard_normal((batch, L))
    ref = cm(F.linear(tm(x), torch.from_numpy(W), torch.from_numpy(b))) + r
    failed = []
    if not np.allclose(oracle.linear(W, x, b, r, lib=lib), ref, rtol=1e-12, atol=1e-12):
        failed.append("linear")
    wide = cm(F.linear(torch.from_numpy(dt)[:, :, None], torch.from_numpy(w[:, None])))
    if not np.allclose(oracle.dt_proj(dt, w, lib=lib), wide, rtol=1e-12, atol=1e-12):
        failed.append("dt_proj")
    return failed


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
def test_unmodified_source_passes_proj_battery(tmp_path, source):
    assert proj_battery(_build(tmp_path, "orig", source)) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(PROJ_MUTATIONS))
def test_proj_mutant_is_caught(tmp_path, source, name):
    old, new = PROJ_MUTATIONS[name]
    assert source.count(old) == 1, "mutation anchor missing: %s" % name
    assert proj_battery(_build(tmp_path, name, source.replace(old, new))), \
        "planted mistake %r passed the projection pins" % name
