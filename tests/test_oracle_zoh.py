"""Pins of the oracle's exact zero-order-hold discretisation. The guide's
section "Discretization via Zero-Order Hold (ZOH)" gives B_bar = (exp(delta
A) - 1) / A * B before approximating it by delta * B. Zero-order hold means
that the input is held constant over each step of length delta_t and the
continuous system dh/dtau = A h + B_t u_t is solved exactly; two independent
references check that:

  * scipy.signal.cont2discrete(method="zoh") for a one-state system at a
    fixed step, filtered with scipy.signal.lfilter;
  * scipy.integrate.solve_ivp integrating the continuous system over every
    step (time-varying delta, B and C).

Plausible mistakes planted in a copy of the oracle must fail them."""
import shutil

import numpy as np
import pytest
import scipy.integrate
import scipy.signal
import scipy.special

import oracle


def softplus(x):
    return np.logaddexp(0.0, x)


@pytest.mark.parametrize("a", [-1.3, -0.02, 0.4])
def test_single_state_matches_cont2discrete(oracle_lib, a):
    rng = np.random.default_rng(71)
    L, dt, b, c, D = 40, 0.37, 0.8, -1.1, 0.3
    u = rng.standard_normal((1, 1, L))
    Ad, Bd, _, _, _ = scipy.signal.cont2discrete((np.array([[a]]), np.array([[b]]),
                                                  np.array([[c]]), np.array([[0.0]])), dt,
                                                 method="zoh")
    ref = scipy.signal.lfilter([c * Bd[0, 0]], [1.0, -Ad[0, 0]], u[0, 0]) + D * u[0, 0]
    got = oracle.s6_1d(u, np.full((1, 1, L), dt), None, np.full((1, 1, L), b),
                       np.full((1, 1, L), c), np.array([[a]]), np.array([D]), None,
                       delta_softplus=False, zoh=True)
    np.testing.assert_allclose(got[0, 0], ref, rtol=1e-12, atol=1e-12)


def ode_reference(u, dl, B, C, A, D, bias):
    """One forward direction, one channel: solve dh/dtau = A h + B_t u_t over
    [0, delta_t] for every step t (u_t, B_t held), then y_t = C_t h + D u_t."""
    L = u.shape[0]
    delta = softplus(dl + bias)
    h = np.zeros(A.shape[0])
    y = np.zeros(L)
    for t in range(L):
        drive = B[:, t] * u[t]
        sol = scipy.integrate.solve_ivp(lambda _, hh: A * hh + drive, (0.0, delta[t]), h,
                                        method="DOP853", rtol=1e-12, atol=1e-14)
        h = sol.y[:, -1]
        y[t] = C[:, t] @ h + D * u[t]
    return y


def ode_case(seed):
    rng = np.random.default_rng(seed)
    N, L = 3, 6
    u = rng.standard_normal(L)
    dl = rng.standard_normal(L)
    B = rng.standard_normal((N, L))
    C = rng.standard_normal((N, L))
    A = np.array([-2.5, -0.3, 0.7])
    D, bias = 0.6, 0.4
    return u, dl, B, C, A, D, bias


def test_matches_ode_integration(oracle_lib):
    u, dl, B, C, A, D, bias = ode_case(72)
    got = oracle.s6_1d(u[None, None], dl[None, None], None, B[None], C[None], A[None],
                       np.array([D]), np.array([bias]), zoh=True)
    np.testing.assert_allclose(got[0, 0], ode_reference(u, dl, B, C, A, D, bias), rtol=1e-9,
                               atol=1e-10)


def test_A_zero_gives_the_delta_B_form(oracle_lib):
    """At A = 0 the hold's limit is delta * B, the code's form."""
    rng = np.random.default_rng(73)
    u, dl, z = (rng.standard_normal((2, 3, 11)) for _ in range(3))
    B, C = rng.standard_normal((2, 4, 11)), rng.standard_normal((2, 4, 11))
    A = np.zeros((2, 3, 4))
    D, bias = rng.standard_normal((2, 3)), rng.standard_normal((2, 3))
    np.testing.assert_array_equal(oracle.vim_bidir(u, dl, z, B, C, A, D, bias, zoh=True),
                                  oracle.vim_bidir(u, dl, z, B, C, A, D, bias))


def test_vim_is_the_gated_sum_of_one_direction_scans(oracle_lib):
    rng = np.random.default_rng(74)
    u, dl, z = (rng.standard_normal((1, 2, 9)) for _ in range(3))
    B, C = rng.standard_normal((1, 4, 9)), rng.standard_normal((1, 4, 9))
    A = -rng.uniform(0.1, 3.0, (2, 2, 4))
    D, bias = rng.standard_normal((2, 2)), rng.standard_normal((2, 2))
    parts = [oracle.s6_1d(u, dl, None, B, C, A[k], D[k], bias[k], reverse=k == 1, zoh=True)
             for k in range(2)]
    ref = (parts[0] + parts[1]) * z * scipy.special.expit(z)
    np.testing.assert_allclose(oracle.vim_bidir(u, dl, z, B, C, A, D, bias, zoh=True), ref,
                               rtol=1e-12, atol=1e-12)


# ---- the pins must be able to fail
ZOH_MUTATIONS = {
    "hold_without_division": ("expm1(A[n] * delta) / A[n]", "expm1(A[n] * delta)"),
    "hold_with_exp": ("expm1(A[n] * delta) / A[n]", "exp(A[n] * delta) / A[n]"),
    "hold_sign": ("expm1(A[n] * delta) / A[n]", "expm1(-A[n] * delta) / A[n]"),
    "hold_ignored": ("if (J->zoh)", "if (0)"),
}


def zoh_battery(lib):
    u, dl, B, C, A, D, bias = ode_case(75)
    try:
        got = oracle.scan(u[None, None], dl[None, None], None, B[None], C[None], A[None, None],
                          np.array([[D]]), np.array([[bias]]), orders=(0,), bc_per_direction=False,
                          lib=lib, nthreads=1, zoh=True)
    except ValueError:
        return ["ode"]
    ok = np.allclose(got[0, 0], ode_reference(u, dl, B, C, A, D, bias), rtol=1e-9, atol=1e-10)
    return [] if ok else ["ode"]


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
def test_unmodified_source_passes_zoh_battery(tmp_path, source):
    assert zoh_battery(_build(tmp_path, "orig", source)) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(ZOH_MUTATIONS))
def test_zoh_mutant_is_caught(tmp_path, source, name):
    old, new = ZOH_MUTATIONS[name]
    assert source.count(old) == 1, "mutation anchor missing: %s" % name
    assert zoh_battery(_build(tmp_path, name, source.replace(old, new))), \
        "planted mistake %r passed the zero-order-hold pins" % name
