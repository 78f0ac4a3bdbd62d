"""fp64 CPU oracle of SS2D with the back half of the VSS block: LayerNorm over the channels of
the merged map, then the gate (TEST INFRASTRUCTURE ONLY; see oracle/__init__.py).

Source: "Vision Mamba structure and principle" (freeymw.com), section 1 -- in the VSS block the
SS2D features are normalised by Layer Normalization and then multiplied elementwise by the other
branch (a linear layer and the activation, SiLU by default) before the output linear layer and
the residual.  The same page's `MambaLayer` code normalises a flattened map with
`nn.LayerNorm(dim)` over the channels of each token, as does the image-classification
walkthrough (mooersco.com, section 3) on channel-last maps: per pixel, over the channel
dimension, biased variance, eps inside the square root, a learned per-channel scale and shift.
Readings taken here: eps = 1e-5 (that layer's default; the pages pass none), and the gate is
out = LN(M) * silu(z), z being the other branch before its activation, as for the SS2D path's
own gate.  The linear layers on either side are not part of this op.
"""
from __future__ import annotations

import numpy as np

from .front_oracle import ss2d_front_bwd, ss2d_front_fwd
from .ss2d_oracle import ss2d_bwd, ss2d_fwd


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def channel_layer_norm(M, w=None, b=None, eps=1e-5, return_stats=False):
    """LayerNorm over axis 1 of a (batch, C, H, W) map: per pixel, mu = mean_c M,
    var = mean_c (M - mu)^2, out = (M - mu) / sqrt(var + eps) * w[c] + b[c]."""
    M = _f64(M)
    mu = M.mean(axis=1, keepdims=True)
    var = ((M - mu) ** 2).mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (M - mu) * rstd
    out = xhat
    if w is not None:
        out = out * _f64(w)[None, :, None, None]
    if b is not None:
        out = out + _f64(b)[None, :, None, None]
    return (out, xhat, rstd) if return_stats else out


def channel_layer_norm_bwd(dy, xhat, rstd, w=None):
    """Gradient of channel_layer_norm w.r.t. M, w and b, given dL/dout = dy and the saved
    normalised map and 1/std: with g = dy * w, dM = rstd * (g - mean_c g - xhat * mean_c(g xhat)),
    dw = sum over (batch, pixels) of dy * xhat, db = sum of dy."""
    dy = _f64(dy)
    g = dy * _f64(w)[None, :, None, None] if w is not None else dy
    dM = rstd * (g - g.mean(axis=1, keepdims=True) - xhat * (g * xhat).mean(axis=1, keepdims=True))
    return dM, np.sum(dy * xhat, axis=(0, 2, 3)), np.sum(dy, axis=(0, 2, 3))


def _merged(x, delta, A, B, C, D, delta_bias, delta_softplus, conv_w, conv_b):
    # the merged four-route sum with its skip term, before any normalisation or gate
    if conv_w is not None:
        return ss2d_front_fwd(x, conv_w, conv_b, delta, A, B, C, D, delta_bias, None, delta_softplus)
    return ss2d_fwd(x, delta, A, B, C, D, delta_bias, None, delta_softplus)


def ss2d_ln_fwd(x, delta, A, B, C, D=None, delta_bias=None, z=None, ln_w=None, ln_b=None, ln_eps=1e-5,
                conv_w=None, conv_b=None, delta_softplus=True):
    """out = channel_layer_norm(M, ln_w, ln_b, ln_eps) * silu(z) (no factor without z), where M is
    the merged SS2D output (optionally after the input front conv_w, conv_b)."""
    M = _merged(x, delta, A, B, C, D, delta_bias, delta_softplus, conv_w, conv_b)
    y = channel_layer_norm(M, ln_w, ln_b, ln_eps)
    return y * _silu(_f64(z)) if z is not None else y


def ss2d_ln_bwd(x, delta, A, B, C, D=None, delta_bias=None, z=None, ln_w=None, ln_b=None, ln_eps=1e-5,
                conv_w=None, conv_b=None, dout=None, delta_softplus=True):
    """Exact gradient of ss2d_ln_fwd: the gate's, the LayerNorm's, then the SS2D (and front)
    gradient of M.  Returns the SS2D dict (dx, ddelta, dA, dB, dC, dD, ddelta_bias, with
    dconv_w/dconv_b under the front) plus dz, dln_w, dln_b (None for absent inputs)."""
    M = _merged(x, delta, A, B, C, D, delta_bias, delta_softplus, conv_w, conv_b)
    y, xhat, rstd = channel_layer_norm(M, ln_w, ln_b, ln_eps, return_stats=True)
    dout = _f64(dout)
    if z is not None:
        zz = _f64(z)
        s = 1.0 / (1.0 + np.exp(-zz))
        dy = dout * zz * s
        dz = dout * y * s * (1.0 + zz * (1.0 - s))
    else:
        dy, dz = dout, None
    dM, dw, db = channel_layer_norm_bwd(dy, xhat, rstd, ln_w)
    if conv_w is not None:
        g = ss2d_front_bwd(x, conv_w, conv_b, delta, A, B, C, D, delta_bias, None, dM, delta_softplus)
    else:
        g = ss2d_bwd(x, delta, A, B, C, D, delta_bias, None, dM, delta_softplus)
    out = dict(g)
    out["dz"] = dz
    out["dln_w"] = dw if ln_w is not None else None
    out["dln_b"] = db if ln_b is not None else None
    return out
