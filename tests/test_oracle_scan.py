"""Pins of the oracle's selective scan (forward) against things other than itself.

* A = 0 turns the scan into a cumulative sum.
* Constant delta/B/C per row gives a geometric series with a closed form.
* A brute-force semiseparable matrix y = M u (no recurrence at all) on small L.
* Impulse response / causality, linearity in u, B = 0 or C = 0 leaving only D*u.
* Group broadcast of B/C and the last state.
* softplus against its asymptotes.
"""
import numpy as np
import pytest

import oracle


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def silu(v):
    return v / (1 + np.exp(-v))


def brute_force(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False):
    """y = M u + D u with M[t, s] = sum_n C_t[n] exp(A[n] (S_t - S_s)) delta_s B_s[n]
    for s <= t (S = cumulative sum of delta), built element by element."""
    batch, dim, L = u.shape
    G = B.shape[1]
    out = np.zeros((batch, dim, L))
    for b in range(batch):
        for d in range(dim):
            g = d // (dim // G)
            dt = delta[b, d] + (delta_bias[d] if delta_bias is not None else 0.0)
            if softplus:
                dt = np.log(1.0 + np.exp(dt))
            S = np.cumsum(dt)
            M = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    M[t, s] = np.sum(C[b, g, :, t] * np.exp(A[d] * (S[t] - S[s])) * dt[s] * B[b, g, :, s])
            y = M @ u[b, d]
            if D is not None:
                y = y + D[d] * u[b, d]
            if z is not None:
                y = y * silu(z[b, d])
            out[b, d] = y
    return out


def test_hand_worked_example():
    # L = 3, N = 1, A = -ln 2 so each step halves the state; delta = 1, B = C = 1, D = 0.
    u = np.array([[[1.0, 0.0, 2.0]]])
    delta = np.ones((1, 1, 3))
    A = np.array([[-np.log(2.0)]])
    B = np.ones((1, 1, 1, 3))
    C = np.ones((1, 1, 1, 3))
    y, last = oracle.ss_fwd(u, delta, A, B, C, return_last_state=True)
    # h0 = 1, h1 = 0.5, h2 = 0.25 + 2 = 2.25
    np.testing.assert_allclose(y[0, 0], [1.0, 0.5, 2.25], rtol=0, atol=1e-15)
    np.testing.assert_allclose(last[0, 0], [2.25], rtol=0, atol=1e-15)


@pytest.mark.parametrize("N,G", [(1, 1), (4, 2), (16, 1)])
def test_A_zero_is_cumsum(N, G):
    batch, dim, L = 2, 4, 37
    u, delta = rnd(1, batch, dim, L), np.abs(rnd(2, batch, dim, L))
    B, C = rnd(3, batch, G, N, L), rnd(4, batch, G, N, L)
    y = oracle.ss_fwd(u, delta, np.zeros((dim, N)), B, C)
    for d in range(dim):
        g = d // (dim // G)
        h = np.cumsum((delta[:, d] * u[:, d])[:, None, :] * B[:, g], axis=-1)  # (batch, N, L)
        np.testing.assert_allclose(y[:, d], np.sum(C[:, g] * h, axis=1), rtol=1e-12, atol=1e-12)


def test_A_zero_scalar_cumsum():
    u, delta = rnd(5, 1, 1, 50), np.abs(rnd(6, 1, 1, 50))
    y = oracle.ss_fwd(u, delta, np.zeros((1, 1)), np.ones((1, 1, 1, 50)), np.ones((1, 1, 1, 50)), D=np.zeros(1))
    np.testing.assert_allclose(y[0, 0], np.cumsum(delta[0, 0] * u[0, 0]), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N", [1, 3, 8])
def test_geometric_closed_form(N):
    L = 60
    rng = np.random.default_rng(N)
    dt = 0.3
    A = -rng.uniform(0.1, 2.0, size=(1, N))
    Bc, Cc = rng.standard_normal(N), rng.standard_normal(N)
    Dd = 0.7
    a = np.exp(dt * A[0])
    B = np.broadcast_to(Bc[None, None, :, None], (1, 1, N, L)).copy()
    C = np.broadcast_to(Cc[None, None, :, None], (1, 1, N, L)).copy()
    # constant input: y_t = u * sum_n C_n dt B_n (1 - a_n^(t+1)) / (1 - a_n) + D u
    u0 = 1.3
    t = np.arange(L)
    y = oracle.ss_fwd(np.full((1, 1, L), u0), np.full((1, 1, L), dt), A, B, C, D=np.array([Dd]))
    ref = u0 * np.sum(Cc[:, None] * dt * Bc[:, None] * (1 - a[:, None] ** (t + 1)) / (1 - a[:, None]), 0) + Dd * u0
    np.testing.assert_allclose(y[0, 0], ref, rtol=1e-12, atol=1e-13)
    # general input: y_t = sum_n C_n dt B_n sum_{s<=t} a_n^(t-s) u_s + D u_t
    u = rng.standard_normal(L)
    y = oracle.ss_fwd(u[None, None], np.full((1, 1, L), dt), A, B, C, D=np.array([Dd]))
    ref = np.array([np.sum(Cc * dt * Bc * np.array([np.sum(a[n] ** (tt - np.arange(tt + 1)) * u[:tt + 1])
                                                    for n in range(N)])) for tt in range(L)]) + Dd * u
    np.testing.assert_allclose(y[0, 0], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("softplus,use_bias,use_z,G", [(False, False, False, 1), (True, True, True, 2),
                                                        (True, False, True, 4), (False, True, False, 1)])
def test_semiseparable_brute_force(softplus, use_bias, use_z, G):
    batch, dim, N, L = 2, 4, 3, 23
    u, delta = rnd(10, batch, dim, L), rnd(11, batch, dim, L)
    if not softplus:
        delta = np.abs(delta)
    A = -np.abs(rnd(12, dim, N))
    B, C = rnd(13, batch, G, N, L), rnd(14, batch, G, N, L)
    D = rnd(15, dim)
    z = rnd(16, batch, dim, L) if use_z else None
    bias = rnd(17, dim) * 0.5 if use_bias else None
    y = oracle.ss_fwd(u, delta, A, B, C, D=D, z=z, delta_bias=bias, delta_softplus=softplus)
    ref = brute_force(u, delta, A, B, C, D=D, z=z, delta_bias=bias, softplus=softplus)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_impulse_response_and_causality():
    L, N, s = 30, 4, 11
    delta = np.abs(rnd(20, 1, 1, L))
    A = -np.abs(rnd(21, 1, N))
    B, C = rnd(22, 1, 1, N, L), rnd(23, 1, 1, N, L)
    u = np.zeros((1, 1, L))
    u[0, 0, s] = 1.0
    y = oracle.ss_fwd(u, delta, A, B, C, D=np.array([0.25]))
    assert (y[0, 0, :s] == 0.0).all()
    S = np.cumsum(delta[0, 0])
    for t in range(s, L):
        m = np.sum(C[0, 0, :, t] * np.exp(A[0] * (S[t] - S[s])) * delta[0, 0, s] * B[0, 0, :, s])
        expect = m + (0.25 if t == s else 0.0)
        assert abs(y[0, 0, t] - expect) <= 1e-13 * max(1.0, abs(expect))


def test_linearity_and_zero_B_or_C():
    batch, dim, N, L = 2, 3, 4, 40
    u1, u2, delta = rnd(30, batch, dim, L), rnd(31, batch, dim, L), rnd(32, batch, dim, L)
    A = -np.abs(rnd(33, dim, N))
    B, C = rnd(34, batch, 1, N, L), rnd(35, batch, 1, N, L)
    D = rnd(36, dim)
    f = lambda uu, BB=B, CC=C: oracle.ss_fwd(uu, delta, A, BB, CC, D=D, delta_softplus=True)
    np.testing.assert_allclose(f(2.5 * u1 - 0.5 * u2), 2.5 * f(u1) - 0.5 * f(u2), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f(u1, BB=np.zeros_like(B)), D[None, :, None] * u1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(f(u1, CC=np.zeros_like(C)), D[None, :, None] * u1, rtol=0, atol=1e-15)


def test_group_broadcast():
    batch, dim, N, L, G = 2, 6, 3, 17, 3
    u, delta = rnd(40, batch, dim, L), rnd(41, batch, dim, L)
    A = -np.abs(rnd(42, dim, N))
    B, C = rnd(43, batch, G, N, L), rnd(44, batch, G, N, L)
    y = oracle.ss_fwd(u, delta, A, B, C, delta_softplus=True)
    per = dim // G
    for g in range(G):
        sl = slice(g * per, (g + 1) * per)
        yg = oracle.ss_fwd(u[:, sl], delta[:, sl], A[sl], B[:, g], C[:, g], delta_softplus=True)
        np.testing.assert_array_equal(y[:, sl], yg)


def test_last_state():
    batch, dim, N, L = 1, 2, 5, 33
    u, delta = rnd(50, batch, dim, L), np.abs(rnd(51, batch, dim, L))
    A = -np.abs(rnd(52, dim, N))
    B, C = rnd(53, batch, 1, N, L), rnd(54, batch, 1, N, L)
    _, last = oracle.ss_fwd(u, delta, A, B, C, return_last_state=True)
    for d in range(dim):
        S = np.cumsum(delta[0, d])
        h = [np.sum(np.exp(A[d, n] * (S[-1] - S)) * delta[0, d] * B[0, 0, n] * u[0, d]) for n in range(N)]
        np.testing.assert_allclose(last[0, d], h, rtol=1e-12, atol=1e-13)


def test_softplus_asymptotes():
    x = np.array([-800.0, -40.0, -5.0, 0.0, 3.0, 40.0, 800.0])
    sp = oracle.softplus(x)
    assert sp[0] == 0.0 or sp[0] < 1e-300
    np.testing.assert_allclose(sp[1], np.exp(-40.0), rtol=1e-15)
    np.testing.assert_allclose(sp[2], np.log(1 + np.exp(-5.0)), rtol=1e-13)  # 1+e^-5 rounds in the reference
    assert sp[3] == np.log(2.0)
    np.testing.assert_allclose(sp[4], np.log(1 + np.exp(3.0)), rtol=1e-15)
    np.testing.assert_allclose(sp[5], 40.0, rtol=1e-15)
    assert sp[6] == 800.0


def test_softplus_path_in_scan():
    # A = 0, N = 1, B = C = 1: y = cumsum(softplus(delta + bias) * u)
    L = 25
    u, delta = rnd(60, 1, 1, L), 3 * rnd(61, 1, 1, L)
    bias = np.array([-1.5])
    y = oracle.ss_fwd(u, delta, np.zeros((1, 1)), np.ones((1, 1, 1, L)), np.ones((1, 1, 1, L)),
                      delta_bias=bias, delta_softplus=True)
    dt = np.log(1 + np.exp(delta[0, 0] + bias[0]))
    np.testing.assert_allclose(y[0, 0], np.cumsum(dt * u[0, 0]), rtol=1e-12, atol=1e-13)
