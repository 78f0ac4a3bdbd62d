"""fp64 CPU oracle of SS2D with its Δ/B/C producer: the per-route input projection and the
low-rank Δ projection computed from the scanned sequence itself (TEST INFRASTRUCTURE ONLY; see
oracle/__init__.py).

Source: "Vision Mamba structure and principle" (freeymw.com), section 2 -- the `Mamba` module
builds x_proj (d_inner -> dt_rank + 2 d_state, no bias) and dt_proj (dt_rank -> d_inner, with
the bias that becomes delta_bias, dt_rank = ceil(d_model / 16)); its forward applies x_proj to
every token of the sequence the scan consumes, splits the result into (dt, B, C), and forms
delta = dt_proj.weight @ dt; the fused `MambaInnerFn` does the same with `F.linear` and a
matrix product.  SS2D runs one such S6 block per route (the SS2D section of the VMamba
translation on blog.csdn.net): here each route k has its own x_proj_w[k] (R + 2N, D) and
dt_proj_w[k] (D, R), applied to route k's scanned sequence.  Readings: the projections act per
token, so route k's (dt, B, C) at step l are those of the pixel route k visits at step l; the
dt_proj bias is the path's delta_bias (added inside the softplus); no intermediate rounding.
"""
from __future__ import annotations

import numpy as np

from .front_oracle import front_bwd, front_fwd
from .ss2d_oracle import cross_merge, cross_scan, ss2d_bwd, ss2d_fwd
from .vss_oracle import channel_layer_norm, channel_layer_norm_bwd


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def route_projections(u, x_proj_w, dt_proj_w):
    """Route k's projections of its scanned sequence xs_k = cross_scan(u)_k (D, L):
    x_dbl_k = x_proj_w[k] @ xs_k (R + 2N, L), dt_k = x_dbl_k[:R], B_k = x_dbl_k[R:R+N],
    C_k = x_dbl_k[R+N:], delta_k = dt_proj_w[k] @ dt_k (D, L).
    Returns xs (Bt,4,D,L), dt (Bt,4,R,L), delta (Bt,4,D,L), B, C (Bt,4,N,L)."""
    Wx, Wdt = _f64(x_proj_w), _f64(dt_proj_w)
    R = Wdt.shape[-1]
    N = (Wx.shape[1] - R) // 2
    xs = cross_scan(_f64(u))
    x_dbl = np.einsum("kcd,bkdl->bkcl", Wx, xs)
    dt, B, C = x_dbl[:, :, :R], x_dbl[:, :, R:R + N], x_dbl[:, :, R + N:]
    delta = np.einsum("kdr,bkrl->bkdl", Wdt, dt)
    return xs, dt, delta, B, C


def ss2d_proj_fwd(x, x_proj_w, dt_proj_w, A, D=None, delta_bias=None, z=None, conv_w=None, conv_b=None,
                  layer_norm=False, ln_w=None, ln_b=None, ln_eps=1e-5, delta_softplus=True):
    """SS2D whose delta, B and C come from route_projections of its input u (u = the input front's
    output when conv_w is given, else x); then the merge, the optional LayerNorm and the gate."""
    u = front_fwd(x, conv_w, conv_b) if conv_w is not None else _f64(x)
    _, _, delta, B, C = route_projections(u, x_proj_w, dt_proj_w)
    M = ss2d_fwd(u, delta, A, B, C, D, delta_bias, None, delta_softplus)
    y = channel_layer_norm(M, ln_w, ln_b, ln_eps) if layer_norm else M
    return y * (_f64(z) / (1.0 + np.exp(-_f64(z)))) if z is not None else y


def ss2d_proj_bwd(x, x_proj_w, dt_proj_w, A, D=None, delta_bias=None, z=None, conv_w=None, conv_b=None,
                  layer_norm=False, ln_w=None, ln_b=None, ln_eps=1e-5, dout=None, delta_softplus=True):
    """Exact gradient of ss2d_proj_fwd (chain rule): the gate's and the LayerNorm's gradients give
    dL/dM; SS2D's gradient gives dL/du (direct path), dL/ddelta, dL/dB, dL/dC; then
    d dt = dt_proj_w^T ddelta, ddt_proj_w = sum ddelta dt^T, dx_dbl = (d dt, dB, dC),
    dx_proj_w = sum dx_dbl xs^T, and the projection path's dL/du = cross_merge(x_proj_w^T dx_dbl).
    Returns dx, dx_proj_w, ddt_proj_w, dA, dD, ddelta_bias, dz, dln_w, dln_b, dconv_w, dconv_b."""
    u = front_fwd(x, conv_w, conv_b) if conv_w is not None else _f64(x)
    Bt, Dm, H, W = u.shape
    Wx, Wdt = _f64(x_proj_w), _f64(dt_proj_w)
    xs, dt, delta, B, C = route_projections(u, Wx, Wdt)
    M = ss2d_fwd(u, delta, A, B, C, D, delta_bias, None, delta_softplus)
    dout = _f64(dout)
    dln_w = dln_b = None
    if layer_norm:
        y, xhat, rstd = channel_layer_norm(M, ln_w, ln_b, ln_eps, return_stats=True)
    else:
        y = M
    if z is not None:
        zz = _f64(z)
        s = 1.0 / (1.0 + np.exp(-zz))
        dy = dout * zz * s
        dz = dout * y * s * (1.0 + zz * (1.0 - s))
    else:
        dy, dz = dout, None
    if layer_norm:
        dM, dw, db = channel_layer_norm_bwd(dy, xhat, rstd, ln_w)
        dln_w = dw if ln_w is not None else None
        dln_b = db if ln_b is not None else None
    else:
        dM = dy
    g = ss2d_bwd(u, delta, A, B, C, D, delta_bias, None, dM, delta_softplus)
    ddelta = g["ddelta"]
    d_dt = np.einsum("kdr,bkdl->bkrl", Wdt, ddelta)
    ddt_proj_w = np.einsum("bkdl,bkrl->kdr", ddelta, dt)
    dx_dbl = np.concatenate([d_dt, g["dB"], g["dC"]], axis=2)
    dx_proj_w = np.einsum("bkcl,bkdl->kcd", dx_dbl, xs)
    du = g["dx"] + cross_merge(np.einsum("kcd,bkcl->bkdl", Wx, dx_dbl), H, W)
    out = {"dx_proj_w": dx_proj_w, "ddt_proj_w": ddt_proj_w, "dA": g["dA"], "dD": g["dD"],
           "ddelta_bias": g["ddelta_bias"], "dz": dz, "dln_w": dln_w, "dln_b": dln_b}
    if conv_w is not None:
        out["dx"], out["dconv_w"], out["dconv_b"] = front_bwd(x, conv_w, conv_b, du)
    else:
        out["dx"] = du
    return out
