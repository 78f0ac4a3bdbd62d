"""Pins of the oracle's bidirectional (Vision Mamba) scan.

* The page's own structure (`bimamba_inner_ref`): two separate scans, the second over the
  flipped x, delta, B, C and gate with its own A, each gated inside the scan, the second
  output flipped back and added.  The oracle's merge-then-gate over direction-ordered inputs
  must give the same values.
* Direction swap: exchanging the two directions' inputs and parameters and reversing the gate
  reverses the output (a flip missing or misplaced anywhere breaks this).
* A single step (L = 1) in closed form.
* Central finite differences of the gradient on every input.
"""
import numpy as np
import pytest

import oracle
from test_oracle_scan import rnd


def _inputs(seed, Bt=2, Dm=3, L=7, N=3, z=True, D=True, bias=True):
    return dict(u=rnd(seed, Bt, 2, Dm, L), delta=rnd(seed + 1, Bt, 2, Dm, L), A=-np.abs(rnd(seed + 2, 2, Dm, N)) - 0.1,
                B=rnd(seed + 3, Bt, 2, N, L), C=rnd(seed + 4, Bt, 2, N, L), D=rnd(seed + 5, 2, Dm) if D else None,
                delta_bias=0.3 * rnd(seed + 6, 2, Dm) if bias else None, z=rnd(seed + 7, Bt, Dm, L) if z else None)


def test_matches_bimamba_inner_ref_structure():
    """Shared x, delta, B, C, D, delta_bias; separate A and A_b (the page's first variant)."""
    Bt, Dm, L, N = 2, 4, 9, 3
    x, delta = rnd(400, Bt, Dm, L), rnd(401, Bt, Dm, L)
    A, A_b = -np.abs(rnd(402, Dm, N)) - 0.1, -np.abs(rnd(403, Dm, N)) - 0.1
    B, C, D, bias, z = rnd(404, Bt, N, L), rnd(405, Bt, N, L), rnd(406, Dm), 0.3 * rnd(407, Dm), rnd(408, Bt, Dm, L)
    flip = lambda a: np.ascontiguousarray(a[..., ::-1])
    y = oracle.ss_fwd(x, delta, A, B, C, D, z=z, delta_bias=bias, delta_softplus=True)
    y_b = oracle.ss_fwd(flip(x), flip(delta), A_b, flip(B), flip(C), D, z=flip(z), delta_bias=bias, delta_softplus=True)
    ref = y + flip(y_b)
    out = oracle.vim_bidir_fwd(np.stack([x, flip(x)], 1), np.stack([delta, flip(delta)], 1), np.stack([A, A_b]),
                               np.stack([B, flip(B)], 1), np.stack([C, flip(C)], 1), np.stack([D, D]),
                               np.stack([bias, bias]), z)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_direction_swap_reverses_output():
    p = _inputs(410)
    out = oracle.vim_bidir_fwd(**p)
    sw = lambda a, ax: None if a is None else np.ascontiguousarray(np.flip(a, ax))
    q = dict(u=sw(p["u"], 1), delta=sw(p["delta"], 1), A=sw(p["A"], 0), B=sw(p["B"], 1), C=sw(p["C"], 1),
             D=sw(p["D"], 0), delta_bias=sw(p["delta_bias"], 0), z=sw(p["z"], -1))
    np.testing.assert_allclose(oracle.vim_bidir_fwd(**q), out[..., ::-1], rtol=1e-12, atol=1e-13)


def test_single_step_closed_form():
    p = _inputs(420, L=1)
    out = oracle.vim_bidir_fwd(**p)
    sp = lambda v: np.log1p(np.exp(v))
    ref = np.zeros(out.shape)
    for k in range(2):
        dt = sp(p["delta"][:, k, :, 0] + p["delta_bias"][k])                     # (Bt, D)
        cb = np.einsum("bn,bn->b", p["C"][:, k, :, 0], p["B"][:, k, :, 0])        # sum_n C_n B_n
        ref[..., 0] += dt * cb[:, None] * p["u"][:, k, :, 0] + p["D"][k] * p["u"][:, k, :, 0]
    z = p["z"]
    np.testing.assert_allclose(out, ref * z / (1 + np.exp(-z)), rtol=1e-12, atol=1e-13)


def _fd(inp, name, dout, eps=1e-6):
    g = np.zeros_like(inp[name])
    flat = g.reshape(-1)
    for i in range(flat.size):
        plus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        minus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        plus[name].reshape(-1)[i] += eps
        minus[name].reshape(-1)[i] -= eps
        flat[i] = (np.sum(dout * oracle.vim_bidir_fwd(**plus)) - np.sum(dout * oracle.vim_bidir_fwd(**minus))) / (2 * eps)
    return g


@pytest.mark.parametrize("case", [dict(), dict(z=False, D=False), dict(bias=False)])
def test_vim_bwd_finite_differences(case):
    p = _inputs(430, Bt=1, Dm=2, L=5, N=2, **case)
    dout = rnd(439, 1, 2, 5)
    g = oracle.vim_bidir_bwd(**p, dout=dout)
    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "delta_bias": "ddelta_bias",
             "z": "dz"}
    for name, gname in names.items():
        if p[name] is None:
            assert g[gname] is None
            continue
        np.testing.assert_allclose(g[gname], _fd(p, name, dout), rtol=1e-6, atol=1e-8, err_msg=name)
