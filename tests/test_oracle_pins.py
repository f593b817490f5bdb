"""Pins of the fp64 oracle to things other than itself.

The source pages print no numeric scan output, so the oracle is pinned by
mathematics: the unrolled closed form of the recurrence (brute force on tiny
inputs), limits with a known answer (delta = 0, A = 0), a first-order IIR
filter (scipy's lfilter), linearity, the impulse response, the time-reversal
identity of the backward pass, and the cross-scan traversal written the way
the page's CrossScan2D code does it (numpy transposes and flips). Each test is
chosen so that a dropped term, a wrong sign or a wrong index in the oracle
fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# independent brute force: y_t = sum_{s<=t} C_t (prod_{r=s+1..t} e^{delta_r A})
#                               delta_s B_s u_s + D u_t
# with the product written as exp(A * sum of deltas) and softplus taken from
# numpy's logaddexp, the gate from scipy's expit.
# ----------------------------------------------------------------------------
def _softplus(x):
    return np.logaddexp(0.0, x)


def brute_direction(u, dl, Bs, Cs, A, D, bias, order, softplus=True):
    """One direction of one (batch, channel) unit.

    u, dl: [L] in token order; Bs, Cs: [N, L] indexed by scan step (already
    arranged in scan order); order: token visited at each step.
    Returns y_k in token order.
    """
    L = len(order)
    x = dl[order] + bias
    delta = _softplus(x) if softplus else x
    uo = u[order]
    y = np.zeros(L)
    for t in range(L):
        acc = 0.0
        for s in range(t + 1):
            decay = np.exp(A * delta[s + 1:t + 1].sum())          # [N]
            acc += np.sum(Cs[:, t] * decay * delta[s] * Bs[:, s]) * uo[s]
        y[order[t]] = acc + D * uo[t]
    return y


def traversal_orders(H, W):
    """Visiting orders of the four VMamba scans, written as the page's
    CrossScan2D does it: a row-major reshape, its flip, the transposed
    (column-major) reshape, and its flip. Entry t is the row-major token id."""
    ids = np.arange(H * W).reshape(H, W)
    s1 = ids.reshape(-1)
    s3 = ids.T.reshape(-1)
    return [s1, s1[::-1].copy(), s3, s3[::-1].copy()]


def brute_vim(u, dl, z, B, C, A, D, bias, softplus=True):
    b_, d_, L = u.shape
    fwd = np.arange(L)
    orders = [fwd, fwd[::-1].copy()]
    y = np.zeros(u.shape)
    for b in range(b_):
        for d in range(d_):
            tot = np.zeros(L)
            for k, od in enumerate(orders):
                Bs = B[b][:, od]
                Cs = C[b][:, od]
                Dk = 0.0 if D is None else D[k, d]
                bk = 0.0 if bias is None else bias[k, d]
                tot += brute_direction(u[b, d], dl[b, d], Bs, Cs, A[k, d], Dk, bk, od, softplus)
            if z is not None:
                tot = tot * z[b, d] * scipy.special.expit(z[b, d])
            y[b, d] = tot
    return y


def brute_cross4(u, dl, z, B, C, A, D, bias, H, W, softplus=True):
    b_, d_, L = u.shape
    orders = traversal_orders(H, W)
    y = np.zeros(u.shape)
    for b in range(b_):
        for d in range(d_):
            tot = np.zeros(L)
            for k, od in enumerate(orders):
                tot += brute_direction(u[b, d], dl[b, d], B[b, k], C[b, k], A[k, d],
                                       D[k, d], bias[k, d], od, softplus)
            if z is not None:
                tot = tot * z[b, d] * scipy.special.expit(z[b, d])
            y[b, d] = tot
    return y


def rand_inputs(rng, batch, dim, N, L, ndir, per_dir_bc=False, gate=True):
    u = rng.standard_normal((batch, dim, L))
    dl = 0.7 * rng.standard_normal((batch, dim, L))
    z = rng.standard_normal((batch, dim, L)) * 2 if gate else None
    bc = (batch, ndir, N, L) if per_dir_bc else (batch, N, L)
    B = rng.standard_normal(bc)
    C = rng.standard_normal(bc)
    # general A: mostly decaying, one state growing, to exercise the sign
    A = -rng.uniform(0.05, 3.0, (ndir, dim, N))
    A[..., -1] = 0.2
    D = rng.standard_normal((ndir, dim))
    bias = rng.uniform(-3.0, 0.5, (ndir, dim))
    return u, dl, z, B, C, A, D, bias


# ----------------------------------------------------------------------------
def test_vim_matches_unrolled_closed_form(oracle_lib):
    rng = np.random.default_rng(7)
    args = rand_inputs(rng, batch=2, dim=3, N=4, L=7, ndir=2)
    ref = brute_vim(*args)
    got = oracle.vim_bidir(*args)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_vim_closed_form_without_softplus_and_gate(oracle_lib):
    rng = np.random.default_rng(8)
    u, dl, z, B, C, A, D, bias = rand_inputs(rng, batch=1, dim=2, N=3, L=6, ndir=2)
    dl = np.abs(dl)
    ref = brute_vim(u, dl, None, B, C, A, D, np.zeros_like(bias), softplus=False)
    got = oracle.vim_bidir(u, dl, None, B, C, A, D, None, delta_softplus=False)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("H,W", [(2, 3), (3, 2), (3, 3)])
def test_cross4_matches_unrolled_closed_form(oracle_lib, H, W):
    rng = np.random.default_rng(100 + 10 * H + W)
    args = rand_inputs(rng, batch=2, dim=2, N=3, L=H * W, ndir=4, per_dir_bc=True)
    ref = brute_cross4(*args, H=H, W=W)
    got = oracle.cross4(*args, H=H, W=W)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_s6_1d_matches_closed_form_both_directions(oracle_lib):
    rng = np.random.default_rng(9)
    u, dl, z, B, C, A, D, bias = rand_inputs(rng, batch=2, dim=2, N=4, L=8, ndir=1)
    for reverse in (False, True):
        od = np.arange(8)[::-1].copy() if reverse else np.arange(8)
        got = oracle.s6_1d(u, dl, z, B, C, A[0], D[0], bias[0], reverse=reverse)
        for b in range(2):
            for d in range(2):
                ref = brute_direction(u[b, d], dl[b, d], B[b][:, od], C[b][:, od], A[0, d],
                                      D[0, d], bias[0, d], od)
                ref = ref * z[b, d] * scipy.special.expit(z[b, d])
                np.testing.assert_allclose(got[b, d], ref, rtol=1e-12, atol=1e-12)


def test_delta_zero_gives_skip_only(oracle_lib):
    """delta = 0 (softplus off, no bias): A_bar = 1, B_bar = 0, h stays 0,
    so y = D u exactly (per direction, summed)."""
    rng = np.random.default_rng(10)
    u, dl, z, B, C, A, D, bias = rand_inputs(rng, batch=2, dim=5, N=16, L=33, ndir=2)
    got = oracle.vim_bidir(u, np.zeros_like(dl), None, B, C, A, D, None, delta_softplus=False)
    exp = (D[0][None, :, None] * u) + (D[1][None, :, None] * u)
    assert np.array_equal(got, exp)


def test_A_zero_is_cumulative_sum(oracle_lib):
    """A = 0: h_t = cumsum of delta B u (numpy.cumsum), y = C_t . h_t + D u."""
    rng = np.random.default_rng(11)
    u, dl, z, B, C, A, D, bias = rand_inputs(rng, batch=2, dim=3, N=5, L=40, ndir=1)
    A0 = np.zeros((3, 5))
    got = oracle.s6_1d(u, dl, None, B, C, A0, D[0], bias[0])
    delta = np.logaddexp(0.0, dl + bias[0][None, :, None])          # [b, d, L]
    incr = delta[:, :, None, :] * B[:, None, :, :] * u[:, :, None, :]  # [b, d, N, L]
    h = np.cumsum(incr, axis=-1)
    ref = np.einsum("bnl,bdnl->bdl", C, h) + D[0][None, :, None] * u
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("a", [-0.7, -5.0, 0.3])
def test_first_order_iir_equals_lfilter(oracle_lib, a):
    """N = 1, constant delta, B = C = 1, D = 0: h_t = e^{delta a} h_{t-1} +
    delta u_t, which is scipy.signal.lfilter([delta], [1, -e^{delta a}], u)."""
    rng = np.random.default_rng(12)
    L = 200
    u = rng.standard_normal((1, 1, L))
    dval = 0.37
    dl = np.full((1, 1, L), dval)
    B = np.ones((1, 1, L))
    C = np.ones((1, 1, L))
    got = oracle.s6_1d(u, dl, None, B, C, np.array([[a]]), np.zeros(1), None,
                       delta_softplus=False)
    ref = scipy.signal.lfilter([dval], [1.0, -np.exp(dval * a)], u[0, 0])
    np.testing.assert_allclose(got[0, 0], ref, rtol=1e-12, atol=1e-12)


def test_softplus_of_delta_matches_logaddexp(oracle_lib):
    """With A = 0, B = C = u = 1, D = 0, y_t is the running sum of delta, so
    the first output is softplus(delta_0 + bias) and the increments are the
    later ones; compared with numpy's logaddexp over a wide argument range."""
    x = np.linspace(-40.0, 40.0, 161)
    L = len(x)
    one = np.ones((1, 1, L))
    got = oracle.s6_1d(one, x[None, None, :] - 0.25, None, np.ones((1, 1, L)),
                       np.ones((1, 1, L)), np.zeros((1, 1)), np.zeros(1), np.array([0.25]))
    sp = np.diff(np.concatenate([[0.0], got[0, 0]]))
    np.testing.assert_allclose(sp, np.logaddexp(0.0, x), rtol=1e-9, atol=1e-15)


def test_linear_in_u(oracle_lib):
    rng = np.random.default_rng(13)
    u, dl, z, B, C, A, D, bias = rand_inputs(rng, batch=2, dim=4, N=16, L=50, ndir=2)
    u2 = rng.standard_normal(u.shape)
    a, b = 1.7, -0.4
    y1 = oracle.vim_bidir(u, dl, z, B, C, A, D, bias)
    y2 = oracle.vim_bidir(u2, dl, z, B, C, A, D, bias)
    y12 = oracle.vim_bidir(a * u + b * u2, dl, z, B, C, A, D, bias)
    np.testing.assert_allclose(y12, a * y1 + b * y2, rtol=1e-10, atol=1e-10)


def test_impulse_response(oracle_lib):
    """u = e_s: y_t = sum_n C_t[n] prod_{r=s+1..t} e^{delta_r A_n} delta_s B_s[n]
    for t >= s, 0 before s (D = 0)."""
    rng = np.random.default_rng(14)
    L, N, s = 30, 6, 11
    u = np.zeros((1, 1, L))
    u[0, 0, s] = 1.0
    dl = 0.5 * rng.standard_normal((1, 1, L))
    B = rng.standard_normal((1, N, L))
    C = rng.standard_normal((1, N, L))
    A = -rng.uniform(0.1, 2.0, (1, N))
    got = oracle.s6_1d(u, dl, None, B, C, A, np.zeros(1), np.array([-1.0]))[0, 0]
    delta = np.logaddexp(0.0, dl[0, 0] - 1.0)
    ref = np.zeros(L)
    for t in range(s, L):
        P = np.ones(N)
        for r in range(s + 1, t + 1):
            P = P * np.exp(delta[r] * A[0])
        ref[t] = np.sum(C[0, :, t] * P * delta[s] * B[0, :, s])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_backward_is_flip_forward_flip(oracle_lib):
    """The backward pass equals the forward scan of the flipped sequence,
    flipped back, with the backward parameters (same values, bit for bit)."""
    rng = np.random.default_rng(15)
    u, dl, z, B, C, A, D, bias = rand_inputs(rng, batch=2, dim=3, N=16, L=45, ndir=1)
    f = lambda a: None if a is None else np.ascontiguousarray(a[..., ::-1])
    back = oracle.s6_1d(u, dl, z, B, C, A[0], D[0], bias[0], reverse=True)
    fwd_flipped = oracle.s6_1d(f(u), f(dl), f(z), f(B), f(C), A[0], D[0], bias[0])
    assert np.array_equal(back, f(fwd_flipped))


def test_vim_is_gated_sum_of_directions(oracle_lib):
    rng = np.random.default_rng(16)
    u, dl, z, B, C, A, D, bias = rand_inputs(rng, batch=2, dim=3, N=16, L=21, ndir=2)
    yb = oracle.vim_bidir(u, dl, z, B, C, A, D, bias)
    f = oracle.s6_1d(u, dl, None, B, C, A[0], D[0], bias[0])
    b = oracle.s6_1d(u, dl, None, B, C, A[1], D[1], bias[1], reverse=True)
    np.testing.assert_allclose(yb, (f + b) * z * scipy.special.expit(z), rtol=1e-13, atol=1e-13)


def test_gate_limits(oracle_lib):
    rng = np.random.default_rng(17)
    u, dl, z, B, C, A, D, bias = rand_inputs(rng, batch=1, dim=2, N=8, L=16, ndir=2)
    assert np.all(oracle.vim_bidir(u, dl, np.zeros_like(u), B, C, A, D, bias) == 0.0)
    ungated = oracle.vim_bidir(u, dl, None, B, C, A, D, bias)
    big = np.full_like(u, 60.0)   # silu(60) = 60 to double precision
    np.testing.assert_allclose(oracle.vim_bidir(u, dl, big, B, C, A, D, bias), 60.0 * ungated,
                               rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("H,W", [(5, 7), (7, 5), (4, 4)])
def test_cross4_traverse_merge_is_four_times_input(oracle_lib, H, W):
    """delta = 0, D_k = 1, no gate: every direction returns u, so the
    cross-merge of the four traversals is exactly 4u (cs_merge o cs_traverse
    = 4x)."""
    rng = np.random.default_rng(18)
    u = rng.standard_normal((2, 3, H * W))
    B = rng.standard_normal((2, 4, 16, H * W))
    y = oracle.cross4(u, np.zeros_like(u), None, B, B, np.full((4, 3, 16), -1.0),
                      np.ones((4, 3)), None, H, W, delta_softplus=False)
    assert np.array_equal(y, 4.0 * u)


@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_cross4_single_direction_isolation(oracle_lib, k):
    """C_j = 0 and D_j = 0 for j != k reduce the cross-scan to one forward
    scan over the k-th traversal (numpy transposes/flips, as in the page's
    CrossScan2D.cs_traverse), mapped back to the grid (cs_merge)."""
    H, W = 5, 7
    L = H * W
    rng = np.random.default_rng(19 + k)
    u, dl, z, B, C, A, D, bias = rand_inputs(rng, batch=2, dim=3, N=16, L=L, ndir=4,
                                             per_dir_bc=True, gate=False)
    for j in range(4):
        if j != k:
            C[:, j] = 0.0
            D[j] = 0.0
    got = oracle.cross4(u, dl, None, B, C, A, D, bias, H, W)
    od = traversal_orders(H, W)[k]
    # forward 1-D scan of the traversed sequence (its B, C already in scan order)
    seq = oracle.s6_1d(u[..., od], dl[..., od], None, B[:, k], C[:, k], A[k], D[k], bias[k])
    ref = np.empty_like(seq)
    ref[..., od] = seq
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_dstate_below_16(oracle_lib):
    """The page's own shape test uses d_state = 8."""
    rng = np.random.default_rng(20)
    args = rand_inputs(rng, batch=1, dim=2, N=8, L=9, ndir=2)
    np.testing.assert_allclose(oracle.vim_bidir(*args), brute_vim(*args), rtol=1e-12, atol=1e-12)


def test_page_shape_examples(oracle_lib):
    """Shapes the pages assert in their verification blocks (golden file):
    the bidirectional block keeps (batch, patches, dim); the cross-scan of a
    (2, 64, 16, 16) map gives four sequences of 256 tokens and merges back."""
    with open(os.path.join(GOLDEN, "page_shapes.json")) as f:
        g = json.load(f)
    vb = g["vim_block"]
    b, L, d = vb["input"]
    rng = np.random.default_rng(21)
    N = vb["d_state"]
    u = rng.standard_normal((b, d, L))
    y = oracle.vim_bidir(u, 0.1 * u, u, rng.standard_normal((b, N, L)),
                         rng.standard_normal((b, N, L)), -np.ones((2, d, N)), np.ones((2, d)),
                         np.zeros((2, d)))
    assert (y.shape[0], y.shape[2], y.shape[1]) == tuple(vb["output"])
    cs = g["cross_scan"]
    b, c, H, W = cs["input"]
    orders = traversal_orders(H, W)
    assert (len(orders), b, len(orders[0]), c) == tuple(cs["traversed"])
    x = rng.standard_normal((b, c, H * W))
    y = oracle.cross4(x, np.zeros_like(x), None, np.zeros((b, 4, 1, H * W)),
                      np.zeros((b, 4, 1, H * W)), np.zeros((4, c, 1)), np.ones((4, c)), None,
                      H, W, delta_softplus=False)
    assert y.reshape(b, c, H, W).shape == tuple(cs["merged"])


def test_bad_arguments_are_rejected(oracle_lib):
    with pytest.raises(ValueError):
        oracle.cross4(np.zeros((1, 1, 6)), np.zeros((1, 1, 6)), None, np.zeros((1, 4, 1, 6)),
                      np.zeros((1, 4, 1, 6)), np.zeros((4, 1, 1)), None, None, H=4, W=2)


def test_threads_do_not_change_results(oracle_lib):
    rng = np.random.default_rng(22)
    args = rand_inputs(rng, batch=3, dim=5, N=16, L=64, ndir=2)
    y1 = oracle.vim_bidir(*args, nthreads=1)
    y8 = oracle.vim_bidir(*args, nthreads=8)
    assert np.array_equal(y1, y8)
