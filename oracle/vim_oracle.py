"""fp64 CPU oracle of Vision Mamba's bidirectional selective scan (TEST INFRASTRUCTURE ONLY;
see oracle/__init__.py).

Source: "Vision Mamba structure and principle" (freeymw.com), section 2 -- `bimamba_inner_ref`
runs one selective scan on the sequence and one on the flipped sequence (its own A, the
flipped delta, B, C and gate) and adds the second output flipped back; the `Mamba` module
with bimamba_type "v2" does the same with a separate set of projections, A, D and dt bias
for the flipped direction.  The Vim article (jsqmd.com) describes the same two-direction
design.

Reading taken here (it covers both variants): every per-direction input -- u, delta, B, C --
is given in that direction's own scan order (direction 1 scans the reversed sequence), with
per-direction A, D and delta_bias; the gate z is one sequence in forward order.  Direction 1's
output is flipped back and added to direction 0's, in fp32 on the GPU, and the sum is gated
once: gating each direction with z in its own order and then adding gives the same value,
since silu(z) is the same factor for both terms.
"""
from __future__ import annotations

import numpy as np

from .ss2d_oracle import ss_bwd, ss_fwd


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _flat(a, shape):
    return None if a is None else np.reshape(_f64(a), shape)


def vim_bidir_fwd(u, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True,
                  return_merged=False):
    """Bidirectional scan forward.

    u, delta: (Bt, 2, D, L) -- direction k in its own order; A: (2, D, N);
    B, C: (Bt, 2, N, L); D, delta_bias: (2, D); z: (Bt, D, L) or None.
    out[b, d, l] = (y0[b, d, l] + y1[b, d, L-1-l]) * silu(z[b, d, l]), where y_k is the
    selective scan (with its D*u term) of direction k.  Returns out (and the pre-gate
    sum on request), fp64.
    """
    u = _f64(u)
    Bt, K, Dm, L = u.shape
    assert K == 2
    N = np.asarray(A).shape[-1]
    # the two directions are the two groups of one generic scan: channel k*D + d reads group k
    ys = ss_fwd(u.reshape(Bt, 2 * Dm, L), _flat(delta, (Bt, 2 * Dm, L)), _flat(A, (2 * Dm, N)), _f64(B), _f64(C),
                D=_flat(D, (2 * Dm,)), z=None, delta_bias=_flat(delta_bias, (2 * Dm,)),
                delta_softplus=delta_softplus).reshape(Bt, 2, Dm, L)
    merged = ys[:, 0] + ys[:, 1, :, ::-1]
    out = merged * _silu(_f64(z)) if z is not None else merged
    return (out, merged) if return_merged else out


def vim_bidir_bwd(u, delta, A, B, C, D=None, delta_bias=None, z=None, dout=None, delta_softplus=True):
    """Exact gradient of vim_bidir_fwd, given dL/dout (Bt, D, L).

    With M the pre-gate sum: dz = dout * M * silu'(z), dM = dout * silu(z); direction 0
    receives dM, direction 1 receives dM flipped (its own order); the rest is the selective
    scan's own gradient.  Returns du, ddelta (Bt,2,D,L), dA (2,D,N), dB, dC (Bt,2,N,L),
    dD, ddelta_bias (2,D) (None when the input is absent) and dz (Bt,D,L) or None.
    """
    u = _f64(u)
    Bt, K, Dm, L = u.shape
    N = np.asarray(A).shape[-1]
    dout = _f64(dout)
    if z is not None:
        _, merged = vim_bidir_fwd(u, delta, A, B, C, D, delta_bias, None, delta_softplus, return_merged=True)
        zz = _f64(z)
        s = 1.0 / (1.0 + np.exp(-zz))
        dmerged = dout * zz * s
        dz = dout * merged * s * (1.0 + zz * (1.0 - s))
    else:
        dmerged, dz = dout, None
    dys = np.stack([dmerged, dmerged[:, :, ::-1]], axis=1).reshape(Bt, 2 * Dm, L)
    g = ss_bwd(u.reshape(Bt, 2 * Dm, L), _flat(delta, (Bt, 2 * Dm, L)), _flat(A, (2 * Dm, N)), _f64(B), _f64(C),
               D=_flat(D, (2 * Dm,)), z=None, delta_bias=_flat(delta_bias, (2 * Dm,)),
               delta_softplus=delta_softplus, dout=np.ascontiguousarray(dys))
    return {
        "du": g["du"].reshape(Bt, 2, Dm, L),
        "ddelta": g["ddelta"].reshape(Bt, 2, Dm, L),
        "dA": g["dA"].reshape(2, Dm, N),
        "dB": g["dB"],
        "dC": g["dC"],
        "dD": None if D is None else g["dD"].reshape(2, Dm),
        "ddelta_bias": None if delta_bias is None else g["ddelta_bias"].reshape(2, Dm),
        "dz": dz,
    }
