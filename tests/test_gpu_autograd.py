"""The autograd wrappers (selective_scan_fn, ss2d, vim_bidir): the gradients autograd produces equal those of
the direct backward calls (which recompute the forward instead of reusing its kept states), the
outputs equal the direct forward's (up to the order of the scan's roundings), absent optionals get
no gradient, and one case is checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ss
from gpu_util import TOL, TOL_GRAD, rel_err, to_dev, to_f64
from selective_scan_amd import synth

pytestmark = pytest.mark.gpu


def _close(a, b, what, tol=1e-6):
    e = rel_err(to_f64(a), to_f64(b))
    assert e <= tol, (what, e)


def _leaf(t):
    return None if t is None else t.detach().clone().requires_grad_(True)


@pytest.mark.parametrize("groups,opt", [(2, True), (0, True), (1, False)], ids=["groups2", "3d-bc", "no-optionals"])
def test_selective_scan_fn_autograd(groups, opt):
    g = torch.Generator().manual_seed(11 + groups)
    batch, dim, L, N = 2, 12, 37, 8
    G = max(groups, 1)
    rnd = lambda *s: torch.randn(*s, generator=g).cuda()
    u, delta = rnd(batch, dim, L), 0.5 * rnd(batch, dim, L)
    A = -(torch.rand(dim, N, generator=g) + 0.2).cuda()
    Bm = rnd(batch, N, L) if groups == 0 else rnd(batch, G, N, L)
    Cm = rnd(batch, N, L) if groups == 0 else rnd(batch, G, N, L)
    D, z, bias = (rnd(dim), rnd(batch, dim, L), 0.1 * rnd(dim)) if opt else (None, None, None)
    dout = rnd(batch, dim, L)
    leaves = [_leaf(t) for t in (u, delta, A, Bm, Cm, D, z, bias)]
    out, last = ss.selective_scan_fn(*leaves, delta_softplus=True, return_last_state=True)
    out.backward(dout)
    ref_out, ref_last = ss.selective_scan_fwd(u, delta, A, Bm, Cm, D=D, z=z, delta_bias=bias, delta_softplus=True,
                                              return_last_state=True)
    _close(out, ref_out, "out")
    _close(last, ref_last, "last_state")
    r = ss.selective_scan_bwd(u, delta, A, Bm, Cm, D=D, z=z, delta_bias=bias, dout=dout, delta_softplus=True)
    for leaf, key in zip(leaves, ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias")):
        if leaf is None:
            assert r[key] is None, key
            continue
        assert leaf.grad.shape == leaf.shape, key
        _close(leaf.grad, r[key], key)


def _ss2d_case(k, ln, proj, seed):
    batch, H, W, dim, N, R = 2, 7, 8, 16, 4, 3
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, "f32", has_z=True, seed_base=seed, with_dout=True)
    t = dict(x=to_dev(inp["x"], "f32"), A=to_dev(inp["A"], "f32"), D=to_dev(inp["D"], "f32"),
             delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], "f32"))
    if proj:
        pw = synth.make_proj_params(dim, N, R, seed_base=seed)
        t.update(delta=None, B=None, C=None, x_proj_w=to_dev(pw["x_proj_w"], "f32"),
                 dt_proj_w=to_dev(pw["dt_proj_w"], "f32"))
    else:
        t.update(delta=to_dev(inp["delta"], "f32"), B=to_dev(inp["B"], "f32"), C=to_dev(inp["C"], "f32"))
    if k:
        fp = synth.make_front_params(dim, k, seed_base=seed)
        t.update(conv_w=to_dev(fp["conv_w"], "f32"), conv_b=to_dev(fp["conv_b"], "f32"))
    if ln:
        lp = synth.make_ln_params(dim, seed_base=seed)
        t.update(layer_norm=True, ln_w=to_dev(lp["ln_w"], "f32"), ln_b=to_dev(lp["ln_b"], "f32"))
    return t, inp, to_dev(inp["dout"], "f32")


GRAD_OF = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "delta_bias": "ddelta_bias",
           "z": "dz", "conv_w": "dconv_w", "conv_b": "dconv_b", "ln_w": "dln_w", "ln_b": "dln_b",
           "x_proj_w": "dx_proj_w", "dt_proj_w": "ddt_proj_w"}


@pytest.mark.parametrize("k,ln,proj", [(0, False, False), (3, True, False), (0, False, True), (3, True, True)],
                         ids=["plain", "front+ln", "producer", "producer+front+ln"])
def test_ss2d_autograd_matches_direct_backward(k, ln, proj):
    t, _, dout = _ss2d_case(k, ln, proj, seed=900 + 10 * k + 2 * ln + proj)
    leaves = {key: _leaf(v) if isinstance(v, torch.Tensor) else v for key, v in t.items()}
    out = ss.ss2d(**leaves)
    out.backward(dout)
    # (the direct forward of the plain case runs as one kernel per plane, whose route scans round
    # in another order than the kept-states forward's)
    _close(out, ss.ss2d_fwd(**t), "out", tol=1e-5)
    r = ss.ss2d_bwd(**t, dout=dout)
    for key, v in leaves.items():
        if not isinstance(v, torch.Tensor):
            continue
        _close(v.grad, r[GRAD_OF[key]], key)


def test_ss2d_autograd_against_oracle():
    t, inp, dout = _ss2d_case(0, False, False, seed=950)
    leaves = {key: _leaf(v) for key, v in t.items()}
    out = ss.ss2d(**leaves)
    out.backward(dout)
    ref = dict(x=inp["x"].astype(np.float64), delta=inp["delta"].astype(np.float64), A=inp["A"].astype(np.float64),
               B=inp["B"].astype(np.float64), C=inp["C"].astype(np.float64), D=inp["D"].astype(np.float64),
               delta_bias=inp["delta_bias"].astype(np.float64), z=inp["z"].astype(np.float64))
    assert rel_err(to_f64(out), oracle.ss2d_fwd(**ref)) <= TOL["f32"]
    g = oracle.ss2d_bwd(**ref, dout=inp["dout"].astype(np.float64))
    for key in ("x", "delta", "A", "B", "C", "D", "delta_bias", "z"):
        assert rel_err(to_f64(leaves[key].grad), g[GRAD_OF[key]]) <= TOL_GRAD, key


def test_vim_bidir_autograd_matches_direct_backward():
    inp = synth.make_vim_inputs(2, 29, 12, 8, "f32", True, 960, True)
    t = dict(u=to_dev(inp["u"], "f32"), delta=to_dev(inp["delta"], "f32"), A=to_dev(inp["A"], "f32"),
             B=to_dev(inp["B"], "f32"), C=to_dev(inp["C"], "f32"), D=to_dev(inp["D"], "f32"),
             delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], "f32"))
    dout = to_dev(inp["dout"], "f32")
    leaves = {k: _leaf(v) for k, v in t.items()}
    out = ss.vim_bidir(**leaves)
    out.backward(dout)
    _close(out, ss.vim_bidir_fwd(**t), "out")
    r = ss.vim_bidir_bwd(**t, dout=dout)
    for key, grad in (("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"), ("D", "dD"),
                      ("delta_bias", "ddelta_bias"), ("z", "dz")):
        _close(leaves[key].grad, r[grad], key)


@pytest.mark.parametrize("k,ln,proj", [(0, False, False), (3, True, True)], ids=["plain", "producer+front+ln"])
def test_ss2d_autograd_repeated_backward(k, ln, proj):
    """Two backwards through one graph (retain_graph=True) give the same gradients: the first
    reuses the forward's kept states, whose workspace the backward then overwrites; the second
    recomputes them."""
    t, _, dout = _ss2d_case(k, ln, proj, seed=970 + k)
    leaves = {key: _leaf(v) if isinstance(v, torch.Tensor) else v for key, v in t.items()}
    out = ss.ss2d(**leaves)
    out.backward(dout, retain_graph=True)
    first = {key: v.grad.clone() for key, v in leaves.items() if isinstance(v, torch.Tensor)}
    for v in leaves.values():
        if isinstance(v, torch.Tensor):
            v.grad = None
    out.backward(dout)
    for key, g1 in first.items():
        assert torch.equal(leaves[key].grad, g1), key


def test_selective_scan_fn_and_vim_repeated_backward():
    """The same for the generic scan and the bidirectional scan."""
    g = torch.Generator().manual_seed(5)
    rnd = lambda *s: torch.randn(*s, generator=g).cuda()
    u, delta, A = rnd(2, 16, 45), 0.5 * rnd(2, 16, 45), -(torch.rand(16, 8, generator=g) + 0.2).cuda()
    Bm, Cm, D, z, bias, dout = rnd(2, 1, 8, 45), rnd(2, 1, 8, 45), rnd(16), rnd(2, 16, 45), 0.1 * rnd(16), rnd(2, 16, 45)
    leaves = [_leaf(x) for x in (u, delta, A, Bm, Cm, D, z, bias)]
    out = ss.selective_scan_fn(*leaves, delta_softplus=True)
    out.backward(dout, retain_graph=True)
    first = [x.grad.clone() for x in leaves]
    for x in leaves:
        x.grad = None
    out.backward(dout)
    for x, g1 in zip(leaves, first):
        assert torch.equal(x.grad, g1)
    inp = synth.make_vim_inputs(2, 29, 12, 8, "f32", True, 961, True)
    vl = {k: _leaf(to_dev(inp[k], "f32")) for k in ("u", "delta", "A", "B", "C", "D", "delta_bias", "z")}
    out = ss.vim_bidir(**vl)
    dout = to_dev(inp["dout"], "f32")
    out.backward(dout, retain_graph=True)
    first = {k: v.grad.clone() for k, v in vl.items()}
    for v in vl.values():
        v.grad = None
    out.backward(dout)
    for k, g1 in first.items():
        assert torch.equal(vl[k].grad, g1), k
