"""Pins of the oracle's SS2D composition.

* An independent composition written with numpy flips/transposes: the route
  k = 2 (k = 3) scan is the ordinary scan over the reversed row-major
  (column-major) sequence, and its result is put back with the inverse moves.
* Gate placement: gating every route with the cross-scanned z and then merging
  equals merging and then gating once per pixel.
* The skip term: sum over routes of D[k, d] * u equals (sum_k D[k, d]) * x.
"""
import numpy as np

import oracle
from test_oracle_scan import rnd


def _inputs(seed, Bt=2, Dm=3, H=4, W=5, N=3):
    L = H * W
    return dict(x=rnd(seed, Bt, Dm, H, W), delta=rnd(seed + 1, Bt, 4, Dm, L),
                A=-np.abs(rnd(seed + 2, 4, Dm, N)), B=rnd(seed + 3, Bt, 4, N, L), C=rnd(seed + 4, Bt, 4, N, L),
                D=rnd(seed + 5, 4, Dm), delta_bias=0.3 * rnd(seed + 6, 4, Dm), z=rnd(seed + 7, Bt, Dm, H, W))


def test_ss2d_vs_flip_transpose_composition():
    p = _inputs(300)
    Bt, Dm, H, W = p["x"].shape
    L = H * W
    out = oracle.ss2d_fwd(**p)
    row = p["x"].reshape(Bt, Dm, L)
    col = np.transpose(p["x"], (0, 1, 3, 2)).reshape(Bt, Dm, L)
    seqs = [row, col, row[..., ::-1], col[..., ::-1]]
    merged = np.zeros((Bt, Dm, H, W))
    for k in range(4):
        y = oracle.ss_fwd(seqs[k], p["delta"][:, k], p["A"][k], p["B"][:, k], p["C"][:, k], D=p["D"][k],
                          delta_bias=p["delta_bias"][k], delta_softplus=True)
        if k >= 2:
            y = y[..., ::-1]
        if k % 2 == 0:
            merged += y.reshape(Bt, Dm, H, W)
        else:
            merged += np.transpose(y.reshape(Bt, Dm, W, H), (0, 1, 3, 2))
    z = p["z"]
    np.testing.assert_allclose(out, merged * z / (1 + np.exp(-z)), rtol=1e-12, atol=1e-13)


def test_gate_per_route_equals_gate_after_merge():
    p = _inputs(310)
    Bt, Dm, H, W = p["x"].shape
    L = H * W
    out = oracle.ss2d_fwd(**p)
    xs = oracle.cross_scan(p["x"]).reshape(Bt, 4 * Dm, L)
    zs = oracle.cross_scan(p["z"]).reshape(Bt, 4 * Dm, L)
    N = p["A"].shape[-1]
    ys = oracle.ss_fwd(xs, p["delta"].reshape(Bt, 4 * Dm, L), p["A"].reshape(4 * Dm, N), p["B"], p["C"],
                       D=p["D"].reshape(-1), z=zs, delta_bias=p["delta_bias"].reshape(-1), delta_softplus=True)
    np.testing.assert_allclose(oracle.cross_merge(ys.reshape(Bt, 4, Dm, L), H, W), out, rtol=1e-12, atol=1e-13)


def test_skip_term_sums_over_routes():
    p = _inputs(320)
    with_D = oracle.ss2d_fwd(**{**p, "z": None})
    no_D = oracle.ss2d_fwd(**{**p, "z": None, "D": None})
    np.testing.assert_allclose(with_D - no_D, p["D"].sum(0)[None, :, None, None] * p["x"], rtol=1e-12, atol=1e-13)


def test_merge_of_ones_is_four():
    H, W = 6, 7
    ones = np.ones((1, 4, 2, H * W))
    assert (oracle.cross_merge(ones, H, W) == 4.0).all()
