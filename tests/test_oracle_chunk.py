"""The chunked form of the scan (P9): the pair operator that joins two pieces of a sequence.

A piece of the recurrence h_t = a_t h_{t-1} + b_t (one state; a_t = exp(delta_t A), b_t =
delta_t B_t u_t, the discretisation of the "Selective scan mechanism" section of the VMamba
translation) acts on the state it starts from as the affine map h -> P h + H, with P the product
of the piece's a_t and H its end state from h = 0.  Running piece 1, then piece 2, is the map
(P1, H1) followed by (P2, H2) = (P2 P1, P2 H1 + H2).  The GPU path splits long sequences into
such pieces when rows are few; these tests pin the operator on the CPU:

* it is associative with identity (1, 0), checked exactly on rationals;
* folding the pieces' maps, computed by the oracle on each piece alone, gives the oracle's own
  end state of the whole sequence, for any split points (P = exp(A * sum of the piece's delta)).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def join(first, second):
    """(P1, H1) then (P2, H2): the affine map of the two pieces run one after the other."""
    P1, H1 = first
    P2, H2 = second
    return (P2 * P1, P2 * H1 + H2)


def _rand_pair(rng):
    f = lambda: Fraction(int(rng.integers(-50, 51)), int(rng.integers(1, 20)))
    return (f(), f())


def test_pair_operator_is_associative_and_has_identity():
    rng = np.random.default_rng(7)
    for _ in range(200):
        p, q, r = _rand_pair(rng), _rand_pair(rng), _rand_pair(rng)
        assert join(join(p, q), r) == join(p, join(q, r))
        assert join((Fraction(1), Fraction(0)), p) == p == join(p, (Fraction(1), Fraction(0)))


def test_pair_operator_is_not_commutative():
    """The order of the pieces matters: a mistake that swapped them would be caught."""
    p, q = (Fraction(1, 2), Fraction(3)), (Fraction(2), Fraction(-1))
    assert join(p, q) != join(q, p)


def _piece_map(u, delta, A, B, C, delta_bias, lo, hi):
    """(P, H) of steps [lo, hi) of one row: H from the oracle's end state on the piece alone."""
    sl = slice(lo, hi)
    H = oracle.ss_fwd(u[:, :, sl], delta[:, :, sl], A, B[..., sl], C[..., sl], delta_bias=delta_bias,
                      delta_softplus=True, return_last_state=True)[1][0, 0]
    dt = oracle.softplus(delta[0, 0, sl] + delta_bias[0])
    P = np.exp(A[0] * dt.sum())
    return P, H


@pytest.mark.parametrize("splits", [[0, 64], [0, 1, 64], [0, 32, 33, 64], [0, 5, 17, 40, 41, 63, 64],
                                    list(range(0, 65, 8))])
def test_folded_pieces_equal_the_whole_sequence(splits):
    rng = np.random.default_rng(len(splits))
    L, N = 64, 6
    u = rng.standard_normal((1, 1, L))
    delta = rng.standard_normal((1, 1, L))
    A = -np.exp(rng.uniform(np.log(1 / 16), np.log(16), size=(1, N)))
    B = rng.standard_normal((1, 1, N, L))
    C = rng.standard_normal((1, 1, N, L))
    bias = np.array([-2.0])
    whole = oracle.ss_fwd(u, delta, A, B, C, delta_bias=bias, delta_softplus=True, return_last_state=True)[1][0, 0]
    acc = (np.ones(N), np.zeros(N))
    for lo, hi in zip(splits[:-1], splits[1:]):
        acc = join(acc, _piece_map(u, delta, A, B, C, bias, lo, hi))
    np.testing.assert_allclose(acc[1], whole, rtol=1e-12, atol=1e-12)
    # grouping the pieces differently (right to left) gives the same map
    acc_r = (np.ones(N), np.zeros(N))
    for lo, hi in reversed(list(zip(splits[:-1], splits[1:]))):
        acc_r = join(_piece_map(u, delta, A, B, C, bias, lo, hi), acc_r)
    np.testing.assert_allclose(acc_r[1], whole, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(acc_r[0], acc[0], rtol=1e-12)
