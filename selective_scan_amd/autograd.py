"""Differentiable wrappers (torch.autograd.Function) over the binding: plumbing only.

`selective_scan_fn` has the interface of the pages' `selective_scan_fn` ("Vision Mamba structure
and principle", section 2: `SelectiveScanFn`): u, delta, A, B, C, D=None, z=None,
delta_bias=None, delta_softplus=False, return_last_state=False; B and C may be 3-D (one group);
the gradient of last_state is not propagated; gradients of absent optionals are None.  `ss2d`
is the fused SS2D op (ss2d_fwd / ss2d_bwd) with its optional input front, LayerNorm and Δ/B/C
producer; `vim_bidir` is Vision Mamba's two-direction scan (vim_bidir_fwd / vim_bidir_bwd).  Each
forward keeps its checkpoint states in a workspace that its backward reuses, so the backward does
not recompute the forward.  Every step runs in the library's kernels.
"""
from __future__ import annotations

import torch

from . import _binding as _bind


class SelectiveScanFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u, delta, A, Bm, Cm, D, z, delta_bias, delta_softplus, return_last_state):
        batch, dim, L = u.shape
        N = A.shape[1]
        G = Bm.shape[1] if Bm.dim() == 4 else 1
        ws = torch.empty(_bind.selective_scan_workspace_bytes(batch, dim, N, L, G), dtype=torch.uint8, device=u.device)
        out, last = _bind.selective_scan_fwd(u, delta, A, Bm, Cm, D=D, z=z, delta_bias=delta_bias,
                                             delta_softplus=delta_softplus, return_last_state=True, workspace=ws)
        ctx.save_for_backward(u, delta, A, Bm, Cm, D, z, delta_bias, ws)
        ctx.delta_softplus = delta_softplus
        ctx.mark_non_differentiable(last)
        return (out, last) if return_last_state else out

    @staticmethod
    def backward(ctx, dout, *unused):  # the gradient of last_state is not propagated
        u, delta, A, Bm, Cm, D, z, delta_bias, ws = ctx.saved_tensors
        g = _bind.selective_scan_bwd(u, delta, A, Bm, Cm, D=D, z=z, delta_bias=delta_bias, dout=dout,
                                     delta_softplus=ctx.delta_softplus, workspace=ws, workspace_has_states=True)
        return (g["du"], g["ddelta"], g["dA"], g["dB"], g["dC"], g["dD"], g["dz"], g["ddelta_bias"], None, None)


def selective_scan_fn(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                      return_last_state=False):
    """Selective scan with autograd: out (and last_state when asked)."""
    return SelectiveScanFn.apply(u, delta, A, B, C, D, z, delta_bias, bool(delta_softplus), bool(return_last_state))


_SS2D_KEYS = ("x", "delta", "A", "B", "C", "D", "delta_bias", "z", "conv_w", "conv_b", "ln_w", "ln_b",
              "x_proj_w", "dt_proj_w")
_SS2D_GRADS = ("dx", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz", "dconv_w", "dconv_b", "dln_w", "dln_b",
               "dx_proj_w", "ddt_proj_w")


class SS2DFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, opts, *tensors):
        kw = dict(zip(_SS2D_KEYS, tensors))
        x, A = kw["x"], kw["A"]
        R = kw["dt_proj_w"].shape[-1] if kw["dt_proj_w"] is not None else 0
        nbytes = _bind.ss2d_workspace_bytes(x.shape[0], x.shape[1], x.shape[2], x.shape[3], A.shape[-1], x.dtype, R)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
        out = _bind.ss2d_fwd(**kw, **opts, workspace=ws, keep_states=True)
        ctx.save_for_backward(*tensors, ws)
        ctx.opts = opts
        ctx.states_valid = True
        return out

    @staticmethod
    def backward(ctx, dout):
        *tensors, ws = ctx.saved_tensors
        kw = dict(zip(_SS2D_KEYS, tensors))
        # ss2d_bwd reuses the workspace's route-output region for its own gradients, so only the
        # first backward finds the forward's states there; a repeated backward (retain_graph)
        # lets the library recompute the forward in the same workspace.
        g = _bind.ss2d_bwd(**kw, **ctx.opts, dout=dout, workspace=ws, workspace_has_states=ctx.states_valid)
        ctx.states_valid = False
        return (None,) + tuple(g.get(k) for k in _SS2D_GRADS)


def ss2d(x, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True, conv_w=None, conv_b=None,
         layer_norm=False, ln_w=None, ln_b=None, ln_eps=1e-5, x_proj_w=None, dt_proj_w=None):
    """Fused SS2D with autograd (arguments as ss2d_fwd); returns out."""
    opts = dict(delta_softplus=bool(delta_softplus), layer_norm=bool(layer_norm), ln_eps=float(ln_eps))
    return SS2DFn.apply(opts, x, delta, A, B, C, D, delta_bias, z, conv_w, conv_b, ln_w, ln_b, x_proj_w, dt_proj_w)


_VIM_KEYS = ("u", "delta", "A", "B", "C", "D", "delta_bias", "z")
_VIM_GRADS = ("du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz")


class VimBidirFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, delta_softplus, *tensors):
        kw = dict(zip(_VIM_KEYS, tensors))
        u, A = kw["u"], kw["A"]
        batch, _, dim, L = u.shape
        ws = torch.empty(_bind.vim_bidir_workspace_bytes(batch, dim, L, A.shape[-1], u.dtype), dtype=torch.uint8,
                         device=u.device)
        out = _bind.vim_bidir_fwd(**kw, delta_softplus=delta_softplus, workspace=ws, keep_states=True)
        ctx.save_for_backward(*tensors, ws)
        ctx.delta_softplus = delta_softplus
        return out

    @staticmethod
    def backward(ctx, dout):
        *tensors, ws = ctx.saved_tensors
        kw = dict(zip(_VIM_KEYS, tensors))
        g = _bind.vim_bidir_bwd(**kw, dout=dout, delta_softplus=ctx.delta_softplus, workspace=ws,
                                workspace_has_states=True)
        return (None,) + tuple(g[k] for k in _VIM_GRADS)


def vim_bidir(u, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True):
    """Vision Mamba's two-direction scan with autograd (arguments as vim_bidir_fwd); returns out."""
    return VimBidirFn.apply(bool(delta_softplus), u, delta, A, B, C, D, delta_bias, z)
