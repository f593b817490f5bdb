"""Pins of the oracle's Vim scan with per-direction inputs. The guide's
BidirectionalVisionMambaBlock ("1. PyTorch Implementation of the
Bidirectional Vision Mamba Block") gives each branch its own conv1d and its
own SimpleSelectiveSSM, whose projections produce that branch's B, C and
delta; so u, delta, B and C exist once per direction. Here they are passed in
token order; the backward branch visits token L-1-t at step t.

The unrolled closed form below builds each direction's scan-ordered B and C
from the token-ordered input itself (no use of the oracle's own flip), and
plausible indexing mistakes planted in a copy of the oracle must fail."""
import shutil

import numpy as np
import pytest
import scipy.special

import oracle
from test_oracle_pins import brute_direction


def dirs_inputs(rng, batch=2, dim=3, N=4, L=9, gate=True):
    u = rng.standard_normal((2, batch, dim, L))
    dl = 0.7 * rng.standard_normal((2, batch, dim, L))
    z = 2 * rng.standard_normal((batch, dim, L)) if gate else None
    B = rng.standard_normal((batch, 2, N, L))
    C = rng.standard_normal((batch, 2, N, L))
    A = -rng.uniform(0.05, 3.0, (2, dim, N))
    A[..., -1] = 0.2
    D = rng.standard_normal((2, dim))
    bias = rng.uniform(-3.0, 0.5, (2, dim))
    return u, dl, z, B, C, A, D, bias


def brute_dirs(u, dl, z, B, C, A, D, bias):
    _, batch, dim, L = u.shape
    fwd = np.arange(L)
    orders = [fwd, fwd[::-1].copy()]
    y = np.zeros((batch, dim, L))
    for b in range(batch):
        for d in range(dim):
            tot = np.zeros(L)
            for k, od in enumerate(orders):
                Bs = B[b, k][:, od]           # step t reads token od[t] of its own copy
                Cs = C[b, k][:, od]
                tot += brute_direction(u[k, b, d], dl[k, b, d], Bs, Cs, A[k, d], D[k, d],
                                       bias[k, d], od)
            if z is not None:
                tot = tot * z[b, d] * scipy.special.expit(z[b, d])
            y[b, d] = tot
    return y


@pytest.mark.parametrize("gate", [True, False])
def test_per_direction_inputs_match_closed_form(oracle_lib, gate):
    rng = np.random.default_rng(51 + gate)
    args = dirs_inputs(rng, gate=gate)
    np.testing.assert_allclose(oracle.vim_dirs(*args), brute_dirs(*args), rtol=1e-11,
                               atol=1e-11)


def test_identical_copies_equal_the_shared_scan(oracle_lib):
    rng = np.random.default_rng(53)
    u, dl, z, B, C, A, D, bias = dirs_inputs(rng)
    u2 = np.stack([u[0], u[0]])
    dl2 = np.stack([dl[0], dl[0]])
    B2 = np.stack([B[:, 0], B[:, 0]], axis=1)
    C2 = np.stack([C[:, 0], C[:, 0]], axis=1)
    np.testing.assert_array_equal(oracle.vim_dirs(u2, dl2, z, B2, C2, A, D, bias),
                                  oracle.vim_bidir(u[0], dl[0], z, B[:, 0], C[:, 0], A, D, bias))


def test_backward_copy_is_isolated(oracle_lib):
    """With the backward read-out off (C_1 = 0, D_1 = 0), the result is the
    forward scan of copy 0 alone: changing copy 1 of u, delta and B changes
    nothing, while changing copy 0 does."""
    rng = np.random.default_rng(54)
    u, dl, z, B, C, A, D, bias = dirs_inputs(rng)
    C[:, 1] = 0.0
    D[1] = 0.0
    y = oracle.vim_dirs(u, dl, z, B, C, A, D, bias)
    u2, dl2, B2 = u.copy(), dl.copy(), B.copy()
    u2[1] += 1.0
    dl2[1] -= 0.5
    B2[:, 1] *= 3.0
    np.testing.assert_array_equal(oracle.vim_dirs(u2, dl2, z, B2, C, A, D, bias), y)
    dl2[0] += 0.25
    assert not np.allclose(oracle.vim_dirs(u2, dl2, z, B2, C, A, D, bias), y)


# ---- the pins must be able to fail
DIRS_MUTATIONS = {
    "delta_shared_not_per_direction": ("((J->per_direction & PER_DIR_DELTA) ? k * copy : 0)", "0"),
    "delta_of_the_other_direction": ("((J->per_direction & PER_DIR_DELTA) ? k * copy : 0)",
                                     "((J->per_direction & PER_DIR_DELTA) ? (1 - k) * copy : 0)"),
}


def dirs_battery(lib):
    rng = np.random.default_rng(4322)
    args = dirs_inputs(rng, batch=1, dim=2, N=3, L=7)
    u, dl, z, B, C, A, D, bias = args
    Bs, Cs = B.copy(), C.copy()
    Bs[:, 1] = B[:, 1, :, ::-1]
    Cs[:, 1] = C[:, 1, :, ::-1]
    try:
        got = oracle.scan(u, dl, z, Bs, Cs, A, D, bias, orders=(0, 1), bc_per_direction=True,
                          u_per_direction=True, delta_per_direction=True, lib=lib, nthreads=2)
    except ValueError:
        return ["dirs"]
    return [] if np.allclose(got, brute_dirs(*args), rtol=1e-10, atol=1e-10) else ["dirs"]


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
def test_unmodified_source_passes_dirs_battery(tmp_path, source):
    assert dirs_battery(_build(tmp_path, "orig", source)) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(DIRS_MUTATIONS))
def test_dirs_mutant_is_caught(tmp_path, source, name):
    old, new = DIRS_MUTATIONS[name]
    assert source.count(old) == 1, "mutation anchor missing: %s" % name
    assert dirs_battery(_build(tmp_path, name, source.replace(old, new))), \
        "planted mistake %r passed the per-direction pins" % name
