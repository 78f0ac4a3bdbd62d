"""Pins of the oracle's back half of the VSS block (LayerNorm over channels of the merged SS2D map,
then the gate).

* channel_layer_norm equals torch's layer_norm applied to the channel-last map (a library routine).
* With unit scale and no shift each pixel's output has mean 0 and mean square var / (var + eps).
* With eps = 0 the normalisation ignores a per-pixel scale a > 0 and shift c of its input.
* With eps = 0 the input gradient of each pixel is orthogonal to the constant vector and to the
  normalised input (LayerNorm's output does not move along either).
* Central finite differences of every gradient of ss2d_ln_fwd, with and without the input front.
"""
import numpy as np
import pytest
import torch

import oracle
from test_oracle_scan import rnd


def test_channel_layer_norm_matches_torch():
    M, w, b = rnd(900, 2, 5, 3, 4) * 3.0 + 1.5, rnd(901, 5), rnd(902, 5)
    got = oracle.channel_layer_norm(M, w, b, eps=1e-5)
    t = torch.from_numpy(M).permute(0, 2, 3, 1)
    ref = torch.nn.functional.layer_norm(t, (5,), torch.from_numpy(w), torch.from_numpy(b), eps=1e-5)
    np.testing.assert_allclose(got, ref.permute(0, 3, 1, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_channel_layer_norm_moments():
    M = rnd(903, 3, 7, 2, 5) * 0.01 + 2.0  # small variance: eps matters
    eps = 1e-5
    y = oracle.channel_layer_norm(M, eps=eps)
    var = M.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).mean(axis=1), var / (var + eps), rtol=1e-10)


def test_channel_layer_norm_scale_shift_invariance():
    M, w, b = rnd(904, 2, 6, 3, 3), rnd(905, 6), rnd(906, 6)
    a = np.exp(rnd(907, 2, 1, 3, 3))
    c = rnd(908, 2, 1, 3, 3) * 5.0
    np.testing.assert_allclose(oracle.channel_layer_norm(a * M + c, w, b, eps=0.0),
                               oracle.channel_layer_norm(M, w, b, eps=0.0), rtol=1e-10, atol=1e-10)


def test_channel_layer_norm_gradient_orthogonality():
    M, w, dy = rnd(909, 2, 6, 3, 3), rnd(910, 6), rnd(911, 2, 6, 3, 3)
    _, xhat, rstd = oracle.channel_layer_norm(M, w, None, eps=0.0, return_stats=True)
    dM, _, _ = oracle.channel_layer_norm_bwd(dy, xhat, rstd, w)
    np.testing.assert_allclose(dM.sum(axis=1), 0.0, atol=1e-10)
    np.testing.assert_allclose((dM * (M - M.mean(axis=1, keepdims=True))).sum(axis=1), 0.0, atol=1e-10)


def _inputs(seed, front, Bt=1, Dm=3, H=3, W=4, N=2, k=3):
    L = H * W
    p = dict(x=rnd(seed, Bt, Dm, H, W), delta=rnd(seed + 1, Bt, 4, Dm, L), A=-np.abs(rnd(seed + 2, 4, Dm, N)) - 0.1,
             B=rnd(seed + 3, Bt, 4, N, L), C=rnd(seed + 4, Bt, 4, N, L), D=rnd(seed + 5, 4, Dm),
             delta_bias=0.3 * rnd(seed + 6, 4, Dm), z=rnd(seed + 7, Bt, Dm, H, W),
             ln_w=1.0 + 0.3 * rnd(seed + 8, Dm), ln_b=0.2 * rnd(seed + 9, Dm))
    if front:
        p.update(conv_w=0.5 * rnd(seed + 10, Dm, k, k), conv_b=0.2 * rnd(seed + 11, Dm))
    return p


@pytest.mark.parametrize("front", [False, True])
def test_ss2d_ln_bwd_finite_differences(front):
    p = _inputs(920 + 20 * front, front)
    dout = rnd(939, 1, 3, 3, 4)
    g = oracle.ss2d_ln_bwd(**p, dout=dout)
    names = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "delta_bias": "ddelta_bias", "z": "dz", "ln_w": "dln_w", "ln_b": "dln_b"}
    if front:
        names.update(conv_w="dconv_w", conv_b="dconv_b")
    eps = 1e-6
    for name, gname in names.items():
        num = np.zeros_like(p[name])
        flat = num.reshape(-1)
        for i in range(flat.size):
            plus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            minus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            plus[name].reshape(-1)[i] += eps
            minus[name].reshape(-1)[i] -= eps
            flat[i] = (np.sum(dout * oracle.ss2d_ln_fwd(**plus)) - np.sum(dout * oracle.ss2d_ln_fwd(**minus))) / (2 * eps)
        np.testing.assert_allclose(g[gname], num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_ss2d_ln_without_gate_or_affine():
    """No gate, unit scale, no shift: the output is the plain normalised merged map."""
    p = _inputs(960, False)
    M = oracle.ss2d_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["delta_bias"], None)
    out = oracle.ss2d_ln_fwd(**{**p, "z": None, "ln_w": None, "ln_b": None})
    mu, sd = M.mean(axis=1, keepdims=True), M.std(axis=1, keepdims=True)
    np.testing.assert_allclose(out * np.sqrt(sd ** 2 + 1e-5) / sd, (M - mu) / sd, rtol=1e-10, atol=1e-10)
