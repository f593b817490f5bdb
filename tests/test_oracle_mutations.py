"""The pins must be able to fail: plant plausible mistakes in a copy of the
oracle (on the CPU), rebuild it, and check that the pin battery rejects every
mutant while accepting the unmodified source."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.signal

import oracle
from test_oracle_pins import brute_cross4, brute_vim, rand_inputs

MUTATIONS = {
    "drop_D_skip": ("yk += Dk * u[p];", "yk += 0.0 * u[p];"),
    "exp_sign": ("exp(delta * A[n])", "exp(-delta * A[n])"),
    "B_token_not_step": ("delta * Bk[n * L + q]", "delta * Bk[n * L + p]"),
    "C_token_not_step": ("Ck[n * L + q]", "Ck[n * L + p]"),
    "column_map_transposed": ("case ORD_COLUMN: return (t % H) * W + t / H;",
                              "case ORD_COLUMN: return (t % W) * H + t / W;"),
    "no_softplus": ("J->delta_softplus ? softplus(x) : x", "x"),
    "no_bias": ("dl[p] + bias", "dl[p]"),
    "sigmoid_gate": ("v *= zz / (1.0 + exp(-zz));", "v *= 1.0 / (1.0 + exp(-zz));"),
    "readout_before_update": ("h[n] = Abar * h[n] + Bbar_x;\n                yk += Ck[n * L + q] * h[n];",
                              "yk += Ck[n * L + q] * h[n];\n                h[n] = Abar * h[n] + Bbar_x;"),
    "state_not_reset": ("for (long n = 0; n < N; ++n) h[n] = 0.0;", ""),
    "B_without_delta": ("delta * Bk[n * L + q] * u[p]", "Bk[n * L + q] * u[p]"),
    "u_at_step_index": ("delta * Bk[n * L + q] * u[p]", "delta * Bk[n * L + q] * u[t]"),
    "softplus_wrong_branch": ("x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x))",
                              "x > 0.0 ? log1p(exp(-x)) : log1p(exp(x))"),
}


def battery(lib):
    """Independent pins; returns the names of the ones that fail."""
    failed = []
    rng = np.random.default_rng(1234)
    args = rand_inputs(rng, batch=1, dim=2, N=3, L=7, ndir=2)
    try:
        got = oracle.scan(*args, orders=(0, 1), bc_per_direction=False, lib=lib, nthreads=2)
        if not np.allclose(got, brute_vim(*args), rtol=1e-10, atol=1e-10):
            failed.append("vim_closed_form")
    except ValueError:
        failed.append("vim_closed_form")
    H, W = 2, 3
    args = rand_inputs(rng, batch=1, dim=2, N=3, L=H * W, ndir=4, per_dir_bc=True)
    try:
        got = oracle.scan(*args, orders=(0, 1, 2, 3), bc_per_direction=True, H=H, W=W, lib=lib)
        if not np.allclose(got, brute_cross4(*args, H=H, W=W), rtol=1e-10, atol=1e-10):
            failed.append("cross4_closed_form")
    except ValueError:
        failed.append("cross4_closed_form")
    # first-order IIR with the softplus off
    L = 50
    u = rng.standard_normal((1, 1, L))
    got = oracle.scan(u, np.full((1, 1, L), 0.3), None, np.ones((1, 1, L)), np.ones((1, 1, L)),
                      np.array([[[-2.0]]]), np.zeros((1, 1)), None, orders=(0,),
                      bc_per_direction=False, delta_softplus=False, lib=lib)
    if not np.allclose(got[0, 0], scipy.signal.lfilter([0.3], [1, -np.exp(-0.6)], u[0, 0]),
                       rtol=1e-10, atol=1e-12):
        failed.append("lfilter")
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
def test_unmodified_source_passes_battery(tmp_path, source):
    assert battery(_build(tmp_path, "orig", source)) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(tmp_path, source, name):
    old, new = MUTATIONS[name]
    assert source.count(old) == 1, "mutation anchor missing: %s" % name
    lib = _build(tmp_path, name, source.replace(old, new))
    assert battery(lib), "planted mistake %r passed every pin" % name
