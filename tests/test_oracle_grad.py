"""Pins of the oracle's gradients: central finite differences in fp64 on every
input, the transpose of the brute-force semiseparable matrix for du, and the
closed forms of dD and dz."""
import numpy as np
import pytest

import oracle
from test_oracle_scan import brute_force, rnd


def _setup(G=2, with_z=True, with_D=True, with_bias=True, softplus=True, L=9):
    batch, dim, N = 2, 4, 3
    inp = dict(u=rnd(100, batch, dim, L), delta=rnd(101, batch, dim, L) * (1.0 if softplus else 0.0)
               + (0.0 if softplus else 0.5 + np.abs(rnd(101, batch, dim, L))),
               A=-np.abs(rnd(102, dim, N)) - 0.2, B=rnd(103, batch, G, N, L), C=rnd(104, batch, G, N, L),
               D=rnd(105, dim) if with_D else None, z=rnd(106, batch, dim, L) if with_z else None,
               delta_bias=0.3 * rnd(107, dim) if with_bias else None)
    dout = rnd(108, batch, dim, L)
    return inp, dout, softplus


def _fd(fun, inp, name, dout, eps=1e-6):
    g = np.zeros_like(inp[name])
    flat = g.reshape(-1)
    for i in range(flat.size):
        plus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        minus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        plus[name].reshape(-1)[i] += eps
        minus[name].reshape(-1)[i] -= eps
        flat[i] = (np.sum(dout * fun(plus)) - np.sum(dout * fun(minus))) / (2 * eps)
    return g


CASES = [dict(G=2), dict(G=1, with_z=False), dict(G=4, with_D=False, with_bias=False),
         dict(G=1, softplus=False, with_bias=False)]


@pytest.mark.parametrize("case", CASES)
def test_ss_bwd_finite_differences(case):
    inp, dout, sp = _setup(**case)
    fun = lambda p: oracle.ss_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                                  delta_bias=p["delta_bias"], delta_softplus=sp)
    g = oracle.ss_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                      delta_bias=inp["delta_bias"], delta_softplus=sp, dout=dout)
    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "delta_bias": "ddelta_bias"}
    for name, gname in names.items():
        if inp[name] is None:
            assert g[gname] is None
            continue
        ref = _fd(fun, inp, name, dout)
        scale = max(1.0, np.abs(ref).max())
        err = np.abs(g[gname] - ref).max() / scale
        assert err < 2e-7, (name, err)


def test_du_is_transpose_of_semiseparable_matrix():
    batch, dim, N, L = 1, 2, 3, 15
    u, delta = rnd(120, batch, dim, L), rnd(121, batch, dim, L)
    A = -np.abs(rnd(122, dim, N))
    B, C = rnd(123, batch, 1, N, L), rnd(124, batch, 1, N, L)
    D, z, dout = rnd(125, dim), rnd(126, batch, dim, L), rnd(127, batch, dim, L)
    g = oracle.ss_bwd(u, delta, A, B, C, D=D, z=z, delta_softplus=True, dout=dout)
    dy = dout * z / (1 + np.exp(-z))
    for d in range(dim):
        # column s of M is the response of y to a unit impulse at s (no gate, no D)
        M = np.zeros((L, L))
        for s in range(L):
            e = np.zeros((batch, dim, L))
            e[0, d, s] = 1.0
            M[:, s] = brute_force(e, delta, A, B, C, softplus=True)[0, d]
        np.testing.assert_allclose(g["du"][0, d] - D[d] * dy[0, d], M.T @ dy[0, d], rtol=1e-11, atol=1e-12)
    # dD = sum over batch and time of dy * u ; dz = dout * (y + D u) * silu'(z)
    np.testing.assert_allclose(g["dD"], np.sum(dy * u, axis=(0, 2)), rtol=1e-12, atol=1e-13)
    _, ypre = oracle.ss_fwd(u, delta, A, B, C, D=D, delta_softplus=True, return_ypre=True)
    s = 1 / (1 + np.exp(-z))
    np.testing.assert_allclose(g["dz"], dout * ypre * s * (1 + z * (1 - s)), rtol=1e-12, atol=1e-13)


def test_ss2d_bwd_finite_differences():
    Bt, Dm, H, W, N = 1, 2, 3, 4, 2
    L = H * W
    inp = dict(x=rnd(200, Bt, Dm, H, W), delta=rnd(201, Bt, 4, Dm, L), A=-np.abs(rnd(202, 4, Dm, N)) - 0.1,
               B=rnd(203, Bt, 4, N, L), C=rnd(204, Bt, 4, N, L), D=rnd(205, 4, Dm),
               delta_bias=0.3 * rnd(206, 4, Dm), z=rnd(207, Bt, Dm, H, W))
    dout = rnd(208, Bt, Dm, H, W)
    fun = lambda p: oracle.ss2d_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["delta_bias"], p["z"])
    g = oracle.ss2d_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["delta_bias"],
                        inp["z"], dout)
    names = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "delta_bias": "ddelta_bias", "z": "dz"}
    for name, gname in names.items():
        ref = _fd(fun, inp, name, dout)
        err = np.abs(g[gname] - ref).max() / max(1.0, np.abs(ref).max())
        assert err < 2e-7, (name, err)
