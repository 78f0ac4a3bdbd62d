"""Pins of the oracle's Δ/B/C producer (per-route x_proj and dt_proj of the scanned sequence).

* The projections equal torch's `F.linear` (x_proj, token-major as the pages call it) and a
  matrix product (dt_proj) applied to each route's sequence.
* The projections act per token: computed on the grid and then laid out in each route's order
  with numpy transposes and flips (no cross_scan), they equal the route-order result.
* Selection weights (dt, B, C copied from input channels, dt_proj of ones) reduce the op to
  plain SS2D with those inputs.
* Central finite differences of every gradient (input, both projection weights, A, D, the Δ
  bias, the gate), also with the input front and the LayerNorm.
"""
import numpy as np
import pytest
import torch

import oracle
from test_oracle_scan import rnd


def _w(seed, D=4, N=2, R=2):
    return 0.4 * rnd(seed, 4, R + 2 * N, D), 0.5 * rnd(seed + 1, 4, D, R)


def test_route_projections_match_torch_linear():
    u = rnd(1500, 2, 4, 3, 5)
    Wx, Wdt = _w(1501)
    xs, dt, delta, B, C = oracle.route_projections(u, Wx, Wdt)
    R, N = 2, 2
    for b in range(2):
        for k in range(4):
            tok = torch.from_numpy(np.ascontiguousarray(xs[b, k].T))  # (L, D) tokens
            x_dbl = torch.nn.functional.linear(tok, torch.from_numpy(Wx[k])).numpy().T  # (R+2N, L)
            np.testing.assert_allclose(dt[b, k], x_dbl[:R], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(B[b, k], x_dbl[R:R + N], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(C[b, k], x_dbl[R + N:], rtol=1e-12, atol=1e-12)
            dref = (torch.from_numpy(Wdt[k]) @ torch.from_numpy(np.ascontiguousarray(x_dbl[:R]))).numpy()
            np.testing.assert_allclose(delta[b, k], dref, rtol=1e-12, atol=1e-12)


def test_projections_are_per_token():
    Bt, D, H, W = 2, 4, 3, 5
    u = rnd(1510, Bt, D, H, W)
    Wx, Wdt = _w(1511)
    _, dt, delta, B, C = oracle.route_projections(u, Wx, Wdt)
    grid = np.einsum("kcd,bdhw->bkchw", Wx, u)                     # every pixel's projections
    orders = [lambda a: a.reshape(*a.shape[:-2], H * W),           # row-major
              lambda a: np.swapaxes(a, -1, -2).reshape(*a.shape[:-2], H * W),  # column-major
              lambda a: a.reshape(*a.shape[:-2], H * W)[..., ::-1],
              lambda a: np.swapaxes(a, -1, -2).reshape(*a.shape[:-2], H * W)[..., ::-1]]
    for k in range(4):
        seq = orders[k](grid[:, k])                                # (Bt, R+2N, L) in route k's order
        np.testing.assert_allclose(dt[:, k], seq[:, :2], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(B[:, k], seq[:, 2:4], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(C[:, k], seq[:, 4:], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(delta[:, k], np.einsum("dr,brl->bdl", Wdt[k], seq[:, :2]), rtol=1e-12,
                                   atol=1e-12)


def test_selection_weights_reduce_to_plain_ss2d():
    Bt, D, H, W, N = 1, 4, 3, 4, 1
    u = rnd(1520, Bt, D, H, W)
    Wx = np.zeros((4, 1 + 2 * N, D))
    Wx[:, 0, 0] = 1.0   # dt = channel 0
    Wx[:, 1, 1] = 1.0   # B = channel 1
    Wx[:, 2, 2] = 1.0   # C = channel 2
    Wdt = np.ones((4, D, 1))
    A = -np.abs(rnd(1521, 4, D, N)) - 0.1
    Dv, bias, z = rnd(1522, 4, D), 0.3 * rnd(1523, 4, D), rnd(1524, Bt, D, H, W)
    xs = oracle.cross_scan(u)
    delta = np.repeat(xs[:, :, 0:1], D, axis=2)
    ref = oracle.ss2d_fwd(u, delta, A, xs[:, :, 1:2], xs[:, :, 2:3], Dv, bias, z)
    got = oracle.ss2d_proj_fwd(u, Wx, Wdt, A, Dv, bias, z)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _inputs(seed, front, ln, Bt=1, D=3, H=3, W=4, N=2, R=2, k=3):
    p = dict(x=rnd(seed, Bt, D, H, W), x_proj_w=0.4 * rnd(seed + 1, 4, R + 2 * N, D),
             dt_proj_w=0.5 * rnd(seed + 2, 4, D, R), A=-np.abs(rnd(seed + 3, 4, D, N)) - 0.1,
             D=rnd(seed + 4, 4, D), delta_bias=0.3 * rnd(seed + 5, 4, D), z=rnd(seed + 6, Bt, D, H, W))
    if front:
        p.update(conv_w=0.5 * rnd(seed + 7, D, k, k), conv_b=0.2 * rnd(seed + 8, D))
    if ln:
        p.update(layer_norm=True, ln_w=1.0 + 0.3 * rnd(seed + 9, D), ln_b=0.2 * rnd(seed + 10, D))
    return p


@pytest.mark.parametrize("front,ln", [(False, False), (True, True)])
def test_ss2d_proj_bwd_finite_differences(front, ln):
    p = _inputs(1530 + 20 * front, front, ln)
    dout = rnd(1549, 1, 3, 3, 4)
    g = oracle.ss2d_proj_bwd(**p, dout=dout)
    names = {"x": "dx", "x_proj_w": "dx_proj_w", "dt_proj_w": "ddt_proj_w", "A": "dA", "D": "dD",
             "delta_bias": "ddelta_bias", "z": "dz"}
    if front:
        names.update(conv_w="dconv_w", conv_b="dconv_b")
    if ln:
        names.update(ln_w="dln_w", ln_b="dln_b")
    eps = 1e-6
    for name, gname in names.items():
        num = np.zeros_like(p[name])
        flat = num.reshape(-1)
        for i in range(flat.size):
            plus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            minus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            plus[name].reshape(-1)[i] += eps
            minus[name].reshape(-1)[i] -= eps
            flat[i] = (np.sum(dout * oracle.ss2d_proj_fwd(**plus)) - np.sum(dout * oracle.ss2d_proj_fwd(**minus))) / (2 * eps)
        np.testing.assert_allclose(g[gname], num, rtol=1e-6, atol=1e-8, err_msg=name)
