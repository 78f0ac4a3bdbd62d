"""Pins of the oracle's SS2D front (depthwise k x k convolution + SiLU before the cross-scan).

* The convolution equals scipy's 2-D cross-correlation of every plane (zero fill, 'same').
* An identity filter (1 at the centre, no bias) reduces the op to SS2D on silu(x).
* Central finite differences of the gradient on x, the filter, its bias and the SS2D inputs.
"""
import numpy as np
import pytest
from scipy.signal import correlate2d

import oracle
from test_oracle_scan import rnd


@pytest.mark.parametrize("k", [1, 3, 5])
def test_dwconv_matches_scipy(k):
    x, w, b = rnd(700, 2, 3, 6, 7), rnd(701, 3, k, k), rnd(702, 3)
    got = oracle.dwconv(x, w, b)
    for bb in range(2):
        for c in range(3):
            ref = correlate2d(x[bb, c], w[c], mode="same", boundary="fill", fillvalue=0.0) + b[c]
            np.testing.assert_allclose(got[bb, c], ref, rtol=1e-12, atol=1e-12)


def _inputs(seed, Bt=1, Dm=2, H=3, W=4, N=2, k=3):
    L = H * W
    return dict(x=rnd(seed, Bt, Dm, H, W), conv_w=0.5 * rnd(seed + 8, Dm, k, k), conv_b=0.2 * rnd(seed + 9, Dm),
                delta=rnd(seed + 1, Bt, 4, Dm, L), A=-np.abs(rnd(seed + 2, 4, Dm, N)) - 0.1,
                B=rnd(seed + 3, Bt, 4, N, L), C=rnd(seed + 4, Bt, 4, N, L), D=rnd(seed + 5, 4, Dm),
                delta_bias=0.3 * rnd(seed + 6, 4, Dm), z=rnd(seed + 7, Bt, Dm, H, W))


def test_identity_filter_reduces_to_ss2d_of_silu():
    p = _inputs(710)
    w = np.zeros_like(p["conv_w"])
    w[:, 1, 1] = 1.0
    out = oracle.ss2d_front_fwd(**{**p, "conv_w": w, "conv_b": None})
    x = p["x"]
    ref = oracle.ss2d_fwd(x / (1 + np.exp(-x)), p["delta"], p["A"], p["B"], p["C"], p["D"], p["delta_bias"], p["z"])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_front_bwd_finite_differences():
    p = _inputs(720)
    dout = rnd(729, 1, 2, 3, 4)
    g = oracle.ss2d_front_bwd(**p, dout=dout)
    names = {"x": "dx", "conv_w": "dconv_w", "conv_b": "dconv_b", "delta": "ddelta", "A": "dA", "B": "dB",
             "C": "dC", "D": "dD", "delta_bias": "ddelta_bias", "z": "dz"}
    eps = 1e-6
    for name, gname in names.items():
        num = np.zeros_like(p[name])
        flat = num.reshape(-1)
        for i in range(flat.size):
            plus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            minus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            plus[name].reshape(-1)[i] += eps
            minus[name].reshape(-1)[i] -= eps
            flat[i] = (np.sum(dout * oracle.ss2d_front_fwd(**plus)) - np.sum(dout * oracle.ss2d_front_fwd(**minus))) / (2 * eps)
        np.testing.assert_allclose(g[gname], num, rtol=1e-6, atol=1e-8, err_msg=name)
