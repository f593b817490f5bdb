"""The algebra behind the chunked scan, pinned on the oracle (CPU, fp64).

The recurrence h_t = exp(delta_t A) h_{t-1} + delta_t B_t u_t is linear in
h, so a run of steps maps its incoming state h to P h + h0 with
P = prod_t exp(delta_t A) = exp(A sum_t delta_t) and h0 the run's end state
from zero, and these aggregates compose associatively in scan order:
(P1, h1) o (P2, h2) = (P1 P2, P2 h1 + h2). The parallel associative scan of
the inferensys glossary "Vision Mamba (Vim)" (item "Parallel Scan
Algorithm") rests on exactly this. Here the oracle's sequential states stand
on both sides: its state after a whole sequence must equal the composition of
the aggregates of any split of it, for the forward and the backward order.
The oracle exposes states through its read-out: with C_t = e_n (one-hot) and
D = 0, y_t is state n after step t."""
import numpy as np

import oracle


def softplus(x):
    return np.logaddexp(0.0, x)


def draw(rng, L, N, dim=3):
    u = rng.standard_normal((1, dim, L))
    dl = 0.5 * rng.standard_normal((1, dim, L))
    B = rng.standard_normal((1, N, L))
    A = -rng.uniform(0.1, 3.0, (dim, N))
    bias = np.log(np.expm1(rng.uniform(0.01, 0.2, dim)))
    return u, dl, B, A, bias


def states(u, dl, B, A, bias, reverse=False):
    """The oracle's state after every step: [dim, N, L] (step order)."""
    dim, N = A.shape
    L = u.shape[-1]
    out = np.empty((dim, N, L))
    for n in range(N):
        C = np.zeros((1, N, L))
        C[0, n] = 1.0
        y = oracle.s6_1d(u, dl, None, B, C, A, np.zeros(dim), bias, reverse=reverse)[0]
        # token p is visited at step p (forward) or L-1-p (backward)
        out[:, n] = y[:, ::-1] if reverse else y
    return out


def aggregate(u, dl, B, A, bias, reverse=False):
    """(P, h0) of a run: P from the sum of delta, h0 from the oracle's scan
    of the run alone, started from zero."""
    S = softplus(dl[0] + bias[:, None]).sum(axis=1)          # [dim]
    P = np.exp(A * S[:, None])                                # [dim, N]
    h0 = states(u, dl, B, A, bias, reverse)[..., -1]
    return P, h0


def compose(x, y):
    (P1, h1), (P2, h2) = x, y
    return P1 * P2, P2 * h1 + h2


def test_split_forward_composes_to_the_whole():
    rng = np.random.default_rng(11)
    u, dl, B, A, bias = draw(rng, 57, 4)
    whole = states(u, dl, B, A, bias)[..., -1]
    for m in (1, 20, 56):
        a = aggregate(u[..., :m], dl[..., :m], B[..., :m], A, bias)
        b = aggregate(u[..., m:], dl[..., m:], B[..., m:], A, bias)
        _, h = compose(a, b)
        np.testing.assert_allclose(h, whole, rtol=1e-12, atol=1e-13)


def test_split_backward_composes_in_reverse_token_order():
    """The backward direction visits the upper tokens first: its carry into
    tokens [0, m) is the aggregate of [m, L) scanned from the top."""
    rng = np.random.default_rng(12)
    u, dl, B, A, bias = draw(rng, 45, 3)
    whole = states(u, dl, B, A, bias, reverse=True)[..., -1]       # state after token 0
    for m in (1, 17, 44):
        upper = aggregate(u[..., m:], dl[..., m:], B[..., m:], A, bias, reverse=True)
        lower = aggregate(u[..., :m], dl[..., :m], B[..., :m], A, bias, reverse=True)
        _, h = compose(upper, lower)
        np.testing.assert_allclose(h, whole, rtol=1e-12, atol=1e-13)
        # the other order is wrong, which the test would notice
        _, h_bad = compose(lower, upper)
        assert np.max(np.abs(h_bad - whole)) > 1e-6


def test_the_carry_restarts_a_chunk_exactly():
    """States inside a chunk = the oracle's scan of the chunk alone plus the
    carried state decayed by the chunk's running product: the replay the
    chunked kernel does."""
    rng = np.random.default_rng(13)
    u, dl, B, A, bias = draw(rng, 40, 4)
    full = states(u, dl, B, A, bias)
    m = 24
    carry = full[..., m - 1]
    local = states(u[..., m:], dl[..., m:], B[..., m:], A, bias)
    cum = np.cumsum(softplus(dl[0, :, m:] + bias[:, None]), axis=1)        # [dim, L - m]
    decay = np.exp(A[:, :, None] * cum[:, None, :])                        # [dim, N, L - m]
    np.testing.assert_allclose(local + decay * carry[..., None], full[..., m:], rtol=1e-12,
                               atol=1e-13)


def test_the_combine_is_associative():
    rng = np.random.default_rng(14)
    for _ in range(20):
        x, y, z = [(rng.uniform(0, 1, 16), rng.standard_normal(16)) for _ in range(3)]
        l = compose(compose(x, y), z)
        r = compose(x, compose(y, z))
        np.testing.assert_allclose(l[0], r[0], rtol=1e-15)
        np.testing.assert_allclose(l[1], r[1], rtol=1e-13, atol=1e-15)
    ident = (np.ones(16), np.zeros(16))
    x = (rng.uniform(0, 1, 16), rng.standard_normal(16))
    for c in (compose(ident, x), compose(x, ident)):
        np.testing.assert_array_equal(c[0], x[0])
        np.testing.assert_array_equal(c[1], x[1])
