"""fp64 CPU oracle of one recurrent step of the selective scan (TEST INFRASTRUCTURE ONLY; see
oracle/__init__.py).

Source: "Vision Mamba structure and principle" (freeymw.com), section 2 -- the `Mamba` module
keeps `ssm_state` (the `last_state` that `selective_scan_fn` returns) between calls and, for
later tokens, advances it one token at a time in place (`self.step`).  The body of `step` is
not printed; the plainest reading, taken here, is one iteration of `selective_scan_ref`'s loop
over t, started from the carried state instead of zero:
  delta = softplus(delta_raw + delta_bias);  h <- exp(delta A) h + delta B x
  y = <C, h> + D x;  out = y * silu(z)
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def ss_step(state, x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False):
    """state (batch, dim, N); x, delta, z (batch, dim); A (dim, N); B, C (batch, G, N) or
    (batch, N) (read as G = 1); D, delta_bias (dim,).  Returns (out (batch, dim), new state)."""
    state, x, delta, A, B, C = map(_f64, (state, x, delta, A, B, C))
    D, z, delta_bias = map(_f64, (D, z, delta_bias))
    if B.ndim == 2:
        B, C = B[:, None], C[:, None]
    batch, dim, N = state.shape
    G = B.shape[1]
    per = dim // G
    new = np.empty_like(state)
    out = np.empty((batch, dim))
    for b in range(batch):
        for d in range(dim):
            g = d // per
            v = delta[b, d] + (delta_bias[d] if delta_bias is not None else 0.0)
            dt = (max(v, 0.0) + np.log1p(np.exp(-abs(v)))) if delta_softplus else v
            y = 0.0
            for n in range(N):
                h = np.exp(dt * A[d, n]) * state[b, d, n] + dt * B[b, g, n] * x[b, d]
                new[b, d, n] = h
                y += C[b, g, n] * h
            if D is not None:
                y += D[d] * x[b, d]
            if z is not None:
                y *= z[b, d] / (1.0 + np.exp(-z[b, d]))
            out[b, d] = y
    return out, new
