"""fp64 CPU oracle of SS2D with its input front: a depthwise k x k convolution and SiLU before
the cross-scan (TEST INFRASTRUCTURE ONLY; see oracle/__init__.py).

Source: "Vision Mamba structure and principle" (freeymw.com), section 1 -- in the VSS block the
SS2D branch passes through a linear layer, a depthwise (separable) convolution and the
activation, SiLU by default, and then into SS2D.  The page gives no kernel size for this 2-D
convolution; taken here: an odd k x k filter per channel with "same" zero padding and a bias
(k = 3 by default on the GPU side).  The linear layer before it is not part of this op.
"""
from __future__ import annotations

import numpy as np

from .ss2d_oracle import ss2d_bwd, ss2d_fwd


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def dwconv(x, w, b=None):
    """Depthwise 'same' cross-correlation: out[b,c,h,w] = bias[c] + sum_{i,j} w[c,i,j] *
    x[b, c, h + i - r, w + j - r] (zero outside the map), r = (k - 1) / 2."""
    x, w = _f64(x), _f64(w)
    Bt, Cc, H, W = x.shape
    k = w.shape[-1]
    r = (k - 1) // 2
    xp = np.zeros((Bt, Cc, H + 2 * r, W + 2 * r))
    xp[:, :, r:r + H, r:r + W] = x
    out = np.zeros((Bt, Cc, H, W))
    for i in range(k):
        for j in range(k):
            out += w[None, :, i, j, None, None] * xp[:, :, i:i + H, j:j + W]
    if b is not None:
        out += _f64(b)[None, :, None, None]
    return out


def _silu(v):
    return v / (1.0 + np.exp(-v))


def ss2d_front_fwd(x, conv_w, conv_b, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True):
    """ss2d_fwd applied to silu(dwconv(x, conv_w, conv_b)); conv_w (D, k, k), conv_b (D,) or None."""
    return ss2d_fwd(_silu(dwconv(x, conv_w, conv_b)), delta, A, B, C, D, delta_bias, z, delta_softplus)


def ss2d_front_bwd(x, conv_w, conv_b, delta, A, B, C, D=None, delta_bias=None, z=None, dout=None,
                   delta_softplus=True):
    """Exact gradient of ss2d_front_fwd: the SS2D gradient w.r.t. its input u = silu(pre),
    pre = dwconv(x), times silu'(pre), then the depthwise convolution's own gradients."""
    g = ss2d_bwd(front_fwd(x, conv_w, conv_b), delta, A, B, C, D, delta_bias, z, dout, delta_softplus)
    dx, dw, db = front_bwd(x, conv_w, conv_b, g["dx"])
    out = dict(g)
    out["dx"] = dx
    out["dconv_w"] = dw
    out["dconv_b"] = db
    return out


def front_fwd(x, conv_w, conv_b):
    """The front alone: u = silu(dwconv(x, conv_w, conv_b))."""
    return _silu(dwconv(x, conv_w, conv_b))


def front_bwd(x, conv_w, conv_b, du):
    """Gradient of front_fwd given dL/du: dpre = du * silu'(pre); dx = the transposed
    convolution of dpre; dw[c,i,j] = sum dpre * x shifted by (i - r, j - r); db = sum dpre."""
    x, w = _f64(x), _f64(conv_w)
    pre = dwconv(x, w, conv_b)
    s = 1.0 / (1.0 + np.exp(-pre))
    dpre = _f64(du) * s * (1.0 + pre * (1.0 - s))
    Bt, Cc, H, W = x.shape
    k = w.shape[-1]
    r = (k - 1) // 2
    xp = np.zeros((Bt, Cc, H + 2 * r, W + 2 * r))
    xp[:, :, r:r + H, r:r + W] = x
    dw = np.zeros_like(w)
    dxp = np.zeros_like(xp)
    for i in range(k):
        for j in range(k):
            dw[:, i, j] = np.sum(dpre * xp[:, :, i:i + H, j:j + W], axis=(0, 2, 3))
            dxp[:, :, i:i + H, j:j + W] += w[None, :, i, j, None, None] * dpre
    return dxp[:, :, r:r + H, r:r + W], dw, (np.sum(dpre, axis=(0, 2, 3)) if conv_b is not None else None)
