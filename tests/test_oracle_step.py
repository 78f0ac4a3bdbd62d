"""Pins of the oracle's single recurrent step.

* Chaining steps from a zero state over a sequence reproduces the C oracle's full scan
  (`ss_fwd`, pinned on its own) step by step, and its last state.
* Starting from a carried state: the scan of a sequence split in two at any point equals the
  scan of the first part followed by steps over the second part.
* A hand-worked single step.
"""
import numpy as np
import pytest

import oracle
from test_oracle_scan import rnd


@pytest.mark.parametrize("G,z,softplus", [(1, True, True), (2, False, True), (1, True, False)])
def test_steps_chain_to_the_scan(G, z, softplus):
    batch, dim, N, L = 2, 4, 3, 6
    u, dl = rnd(500, batch, dim, L), rnd(501, batch, dim, L)
    if not softplus:
        dl = 0.2 + np.abs(dl)
    A, B, C = -np.abs(rnd(502, dim, N)) - 0.1, rnd(503, batch, G, N, L), rnd(504, batch, G, N, L)
    D, zz, bias = rnd(505, dim), rnd(506, batch, dim, L) if z else None, 0.3 * rnd(507, dim) if softplus else None
    ref, last = oracle.ss_fwd(u, dl, A, B, C, D, z=zz, delta_bias=bias, delta_softplus=softplus, return_last_state=True)
    state = np.zeros((batch, dim, N))
    for t in range(L):
        out, state = oracle.ss_step(state, u[..., t], dl[..., t], A, B[..., t], C[..., t], D,
                                    z=None if zz is None else zz[..., t], delta_bias=bias, delta_softplus=softplus)
        np.testing.assert_allclose(out, ref[..., t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(state, last, rtol=1e-12, atol=1e-13)


def test_split_sequence_continues_from_the_state():
    batch, dim, N, L, cut = 1, 3, 4, 9, 5
    u, dl = rnd(510, batch, dim, L), rnd(511, batch, dim, L)
    A, B, C, D = -np.abs(rnd(512, dim, N)) - 0.1, rnd(513, batch, 1, N, L), rnd(514, batch, 1, N, L), rnd(515, dim)
    full = oracle.ss_fwd(u, dl, A, B, C, D, delta_softplus=True)
    _, state = oracle.ss_fwd(u[..., :cut], dl[..., :cut], A, B[..., :cut], C[..., :cut], D, delta_softplus=True,
                             return_last_state=True)
    for t in range(cut, L):
        out, state = oracle.ss_step(state, u[..., t], dl[..., t], A, B[..., t], C[..., t], D, delta_softplus=True)
        np.testing.assert_allclose(out, full[..., t], rtol=1e-12, atol=1e-13)


def test_hand_worked_step():
    # one channel, two states: dt = 0.5 (no softplus), A = (-1, -2), state = (1, -1), B = (2, 1),
    # C = (1, 3), x = 4, D = 0.5:  h = (e^-0.5 + 0.5*2*4, -e^-1 + 0.5*1*4), y = h0 + 3 h1 + 2
    out, h = oracle.ss_step(np.array([[[1.0, -1.0]]]), np.array([[4.0]]), np.array([[0.5]]), np.array([[-1.0, -2.0]]),
                            np.array([[2.0, 1.0]]), np.array([[1.0, 3.0]]), np.array([0.5]))
    h0, h1 = np.exp(-0.5) + 4.0, -np.exp(-1.0) + 2.0
    np.testing.assert_allclose(h[0, 0], [h0, h1], rtol=1e-15)
    np.testing.assert_allclose(out[0, 0], h0 + 3 * h1 + 2.0, rtol=1e-15)
