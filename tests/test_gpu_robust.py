"""Robustness of the HIP path, through the C ABI:

* guard bands: every output (and the workspace) of every entry point sits between bands of a
  known byte pattern; after the call the bands are untouched, and the outputs equal, bit for bit,
  those of the same call on plain buffers (ragged shapes: partial tiles, odd element counts);
* NaN and Inf inputs propagate: the pattern of non-finite outputs equals the fp64 oracle's (NaN
  exactly; with an Inf input, which values are non-finite);
* chunk invariance (the pair operator of the chunked scan): a launch whose few rows make the
  scan split the sequence over wavefronts gives what a launch with enough rows to run each row
  whole gives, image for image.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ss
from gpu_util import TOL, f64, rel_err, to_dev, to_f64
from selective_scan_amd import _binding as bnd
from selective_scan_amd import synth

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


class Guarded:
    """A device tensor with GUARD bytes of PATTERN right before its first and after its last byte."""

    def __init__(self, shape, dtype, init=None):
        n = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((GUARD + n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(shape)
        if init is not None:
            self.t.copy_(init)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.t.data_ptr())

    def intact(self):
        return bool((self.buf[:GUARD] == PATTERN).all()) and bool((self.buf[GUARD + self.n:] == PATTERN).all())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t):
    return bnd.DTYPE_F32 if t.dtype == torch.float32 else bnd.DTYPE_BF16


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_all(guarded, reference):
    torch.cuda.synchronize()
    for name, g in guarded.items():
        assert g.intact(), f"{name}: guard band overwritten"
        if name in reference and reference[name] is not None:
            assert torch.equal(g.t, reference[name]), f"{name}: differs from the plain call"


# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_guard_cross_scan_merge(dtype):
    B, C, H, W = 2, 3, 7, 9
    x = to_dev(synth._normal(1, (B, C, H, W), dtype), dtype)
    xs = Guarded((B, 4, C, H * W), x.dtype)
    assert bnd.lib().ss2d_cross_scan(_p(x), xs.ptr, B, C, H, W, _dt(x), _stream()) == 0
    _check_all({"xs": xs}, {"xs": ss.ss2d_cross_scan(x)})
    y = Guarded((B, C, H, W), x.dtype)
    assert bnd.lib().ss2d_cross_merge(xs.ptr, y.ptr, B, C, H, W, _dt(x), _stream()) == 0
    _check_all({"y": y}, {"y": ss.ss2d_cross_merge(xs.t, H, W)})


SCAN_GUARD_CASES = [
    # batch, dim, N, L, G, dtype
    (2, 24, 16, 77, 2, "bf16"),    # ragged tile, partial wavefront, odd element counts
    (1, 40, 4, 129, 1, "f32"),
    (1, 16, 8, 3000, 1, "f32"),    # few rows: the sequence is chunked
    (3, 5, 1, 33, 1, "bf16"),
]


def _ss_inputs(batch, dim, N, L, G, dtype, seed):
    inp = synth.make_ss_inputs(batch, dim, N, L, G, dtype, has_z=True, seed_base=seed, with_dout=True)
    t = {k: to_dev(inp[k], dtype) for k in ("u", "delta", "B", "C", "z", "dout")}
    t.update(A=to_dev(inp["A"], "f32"), D=to_dev(inp["D"], "f32"), delta_bias=to_dev(inp["delta_bias"], "f32"))
    return t


@pytest.mark.parametrize("case", SCAN_GUARD_CASES, ids=str)
def test_guard_selective_scan(case):
    batch, dim, N, L, G, dtype = case
    t = _ss_inputs(batch, dim, N, L, G, dtype, seed=2100 + L)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True)
    ref_out, ref_last = ss.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], **kw, return_last_state=True)
    ref_g = ss.selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], **kw, dout=t["dout"])
    nbytes = ss.selective_scan_workspace_bytes(batch, dim, N, L, G)
    for with_ws in (True, False):
        out = Guarded(t["u"].shape, t["u"].dtype)
        last = Guarded((batch, dim, N), torch.float32)
        ws = Guarded((nbytes,), torch.uint8) if with_ws else None
        a = bnd.SsFwdArgs(u=_p(t["u"]), delta=_p(t["delta"]), A=_p(t["A"]), Bm=_p(t["B"]), Cm=_p(t["C"]),
                          Dskip=_p(t["D"]), z=_p(t["z"]), delta_bias=_p(t["delta_bias"]), out=out.ptr,
                          last_state=last.ptr, workspace=ws.ptr if ws else None,
                          workspace_bytes=nbytes if ws else 0, batch=batch, dim=dim, dstate=N, seqlen=L,
                          ngroups=G, dtype=_dt(t["u"]), delta_softplus=1)
        assert bnd.lib().selective_scan_fwd(ctypes.byref(a), _stream()) == 0
        gd = {"out": out, "last_state": last}
        if ws:
            gd["workspace"] = ws
            _check_all(gd, {"out": ref_out, "last_state": ref_last})
        else:  # without a workspace a few-row call runs its rows whole: the same result up to rounding order
            _check_all(gd, {})
            assert rel_err(to_f64(out.t), to_f64(ref_out)) <= (1e-5 if dtype == "f32" else 8e-3)
            assert rel_err(to_f64(last.t), to_f64(ref_last)) <= 1e-5
    outs = {"du": t["u"].shape, "ddelta": t["u"].shape, "dz": t["u"].shape, "dB": t["B"].shape, "dC": t["C"].shape}
    g = {k: Guarded(s, t["u"].dtype) for k, s in outs.items()}
    g.update(dA=Guarded((dim, N), torch.float32), dD=Guarded((dim,), torch.float32),
             ddelta_bias=Guarded((dim,), torch.float32), workspace=Guarded((nbytes,), torch.uint8))
    a = bnd.SsBwdArgs(u=_p(t["u"]), delta=_p(t["delta"]), A=_p(t["A"]), Bm=_p(t["B"]), Cm=_p(t["C"]),
                      Dskip=_p(t["D"]), z=_p(t["z"]), delta_bias=_p(t["delta_bias"]), dout=_p(t["dout"]),
                      du=g["du"].ptr, ddelta=g["ddelta"].ptr, dA=g["dA"].ptr, dBm=g["dB"].ptr, dCm=g["dC"].ptr,
                      dDskip=g["dD"].ptr, dz=g["dz"].ptr, ddelta_bias=g["ddelta_bias"].ptr,
                      workspace=g["workspace"].ptr, workspace_bytes=nbytes, workspace_has_states=0, batch=batch,
                      dim=dim, dstate=N, seqlen=L, ngroups=G, dtype=_dt(t["u"]), delta_softplus=1)
    assert bnd.lib().selective_scan_bwd(ctypes.byref(a), _stream()) == 0
    _check_all(g, ref_g)


SS2D_GUARD_CASES = [
    # batch, H, W, dim, N, dtype, front k, layer norm, dt_rank
    (2, 7, 9, 20, 16, "bf16", 0, False, 0),   # staged path, L % 4 != 0
    (2, 8, 8, 5, 4, "f32", 0, False, 0),      # one kernel per plane
    (1, 64, 64, 6, 16, "f32", 0, False, 0),   # chunked route scans
    (1, 9, 11, 24, 16, "bf16", 3, True, 0),   # front and LayerNorm
    (2, 7, 8, 16, 4, "f32", 3, True, 3),      # the producer with front and LayerNorm
    (1, 13, 15, 12, 8, "bf16", 0, False, 2),  # the producer alone, bf16
    (2, 12, 8, 13, 16, "bf16", 0, False, 0),  # route outputs in 4-step blocks, a partial channel block
    (1, 8, 12, 9, 16, "f32", 3, True, 0),     # the same layout with front and LayerNorm
]


@pytest.mark.parametrize("case", SS2D_GUARD_CASES, ids=str)
def test_guard_ss2d(case):
    batch, H, W, dim, N, dtype, k, ln, R = case
    L = H * W
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, dtype, has_z=True, seed_base=2200 + L + k + R, with_dout=True)
    t = dict(x=to_dev(inp["x"], dtype), A=to_dev(inp["A"], "f32"), D=to_dev(inp["D"], "f32"),
             delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dtype))
    if R:
        pw = synth.make_proj_params(dim, N, R, seed_base=2200 + L)
        t.update(delta=None, B=None, C=None, x_proj_w=to_dev(pw["x_proj_w"], "f32"),
                 dt_proj_w=to_dev(pw["dt_proj_w"], "f32"))
    else:
        t.update(delta=to_dev(inp["delta"], dtype), B=to_dev(inp["B"], dtype), C=to_dev(inp["C"], dtype),
                 x_proj_w=None, dt_proj_w=None)
    if k:
        fp = synth.make_front_params(dim, k, seed_base=2200 + L)
        t.update(conv_w=to_dev(fp["conv_w"], "f32"), conv_b=to_dev(fp["conv_b"], "f32"))
    else:
        t.update(conv_w=None, conv_b=None)
    if ln:
        lp = synth.make_ln_params(dim, seed_base=2200 + L)
        t.update(ln_w=to_dev(lp["ln_w"], "f32"), ln_b=to_dev(lp["ln_b"], "f32"))
    else:
        t.update(ln_w=None, ln_b=None)
    dout = to_dev(inp["dout"], dtype)
    kw = dict(t, layer_norm=ln)
    ref_out = ss.ss2d_fwd(**kw)
    ref_g = ss.ss2d_bwd(**kw, dout=dout)
    nbytes = ss.ss2d_workspace_bytes(batch, dim, H, W, N, t["x"].dtype, R)
    common = dict(x=_p(t["x"]), delta=_p(t["delta"]), A=_p(t["A"]), Bm=_p(t["B"]), Cm=_p(t["C"]), Dskip=_p(t["D"]),
                  delta_bias=_p(t["delta_bias"]), z=_p(t["z"]), workspace_bytes=nbytes, batch=batch, dim=dim,
                  height=H, width=W, dstate=N, dtype=_dt(t["x"]), delta_softplus=1, conv_w=_p(t["conv_w"]),
                  conv_b=_p(t["conv_b"]), conv_k=k, layer_norm=int(ln), ln_w=_p(t["ln_w"]), ln_b=_p(t["ln_b"]),
                  ln_eps=1e-5, x_proj_w=_p(t["x_proj_w"]), dt_proj_w=_p(t["dt_proj_w"]), dt_rank=R)
    out, ws = Guarded(t["x"].shape, t["x"].dtype), Guarded((nbytes,), torch.uint8)
    a = bnd.SS2DFwdArgs(**common, out=out.ptr, workspace=ws.ptr, keep_states=0)
    assert bnd.lib().ss2d_fwd(ctypes.byref(a), _stream()) == 0
    _check_all({"out": out, "workspace": ws}, {"out": ref_out})
    shapes = {"dx": (t["x"].shape, t["x"].dtype), "dz": (t["x"].shape, t["x"].dtype),
              "dA": (t["A"].shape, torch.float32), "dD": (t["D"].shape, torch.float32),
              "ddelta_bias": (t["D"].shape, torch.float32)}
    if R:
        shapes.update(dx_proj_w=(t["x_proj_w"].shape, torch.float32), ddt_proj_w=(t["dt_proj_w"].shape, torch.float32))
    else:
        shapes.update(ddelta=(t["delta"].shape, t["x"].dtype), dB=(t["B"].shape, t["x"].dtype),
                      dC=(t["C"].shape, t["x"].dtype))
    if k:
        shapes.update(dconv_w=(t["conv_w"].shape, torch.float32), dconv_b=(t["conv_b"].shape, torch.float32))
    if ln:
        shapes.update(dln_w=((dim,), torch.float32), dln_b=((dim,), torch.float32))
    g = {key: Guarded(s, d) for key, (s, d) in shapes.items()}
    g["workspace"] = Guarded((nbytes,), torch.uint8)
    gp = lambda key: g[key].ptr if key in g else None
    b = bnd.SS2DBwdArgs(**common, dout=_p(dout), dx=gp("dx"), ddelta=gp("ddelta"), dA=gp("dA"), dBm=gp("dB"),
                        dCm=gp("dC"), dDskip=gp("dD"), ddelta_bias=gp("ddelta_bias"), dz=gp("dz"),
                        workspace=g["workspace"].ptr, workspace_has_states=0, dconv_w=gp("dconv_w"),
                        dconv_b=gp("dconv_b"), dln_w=gp("dln_w"), dln_b=gp("dln_b"), dx_proj_w=gp("dx_proj_w"),
                        ddt_proj_w=gp("ddt_proj_w"))
    assert bnd.lib().ss2d_bwd(ctypes.byref(b), _stream()) == 0
    _check_all(g, ref_g)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ss2d_misaligned_io(dtype):
    """x, z and out one element past an aligned address (H, W multiples of 4, N = 16): the route
    scans then load and store element by element, still in the 4-step route blocks, and the merge
    reads and writes the map element by element; the result equals, bit for bit, that of the same
    call on aligned buffers, and nothing around the shifted output is written."""
    batch, H, W, dim, N = 2, 8, 12, 9, 16
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, dtype, has_z=True, seed_base=2400)
    t = dict(x=to_dev(inp["x"], dtype), delta=to_dev(inp["delta"], dtype), A=to_dev(inp["A"], "f32"),
             B=to_dev(inp["B"], dtype), C=to_dev(inp["C"], dtype), D=to_dev(inp["D"], "f32"),
             delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dtype))
    ref = ss.ss2d_fwd(**t)

    def shifted(a):  # a copy of a that starts one element past an aligned address
        buf = torch.empty(a.numel() + 1, dtype=a.dtype, device="cuda")
        v = buf[1:].view(a.shape)
        v.copy_(a)
        return v

    x1, z1 = shifted(t["x"]), shifted(t["z"])
    out = Guarded((t["x"].numel() + 1,), t["x"].dtype, init=torch.zeros(t["x"].numel() + 1, dtype=t["x"].dtype))
    out1 = out.t[1:].view(t["x"].shape)
    nbytes = ss.ss2d_workspace_bytes(batch, dim, H, W, N, t["x"].dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a = bnd.SS2DFwdArgs(x=_p(x1), delta=_p(t["delta"]), A=_p(t["A"]), Bm=_p(t["B"]), Cm=_p(t["C"]),
                        Dskip=_p(t["D"]), delta_bias=_p(t["delta_bias"]), z=_p(z1), out=_p(out1), workspace=_p(ws),
                        workspace_bytes=nbytes, batch=batch, dim=dim, height=H, width=W, dstate=N,
                        dtype=_dt(t["x"]), delta_softplus=1, keep_states=0, conv_k=0, layer_norm=0, ln_eps=1e-5,
                        dt_rank=0)
    assert bnd.lib().ss2d_fwd(ctypes.byref(a), _stream()) == 0
    torch.cuda.synchronize()
    assert out.intact()
    assert float(out.t[0]) == 0.0
    assert torch.equal(out1, ref)


def _shifted_copy(a):
    """A copy of `a` that starts one element past an aligned address."""
    buf = torch.empty(a.numel() + 1, dtype=a.dtype, device="cuda")
    v = buf[1:].view(a.shape)
    v.copy_(a)
    return v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shift", ["dbdc", "gate"])
def test_ss2d_bwd_misaligned(dtype, shift):
    """H, W multiples of 4, N = 16, with some buffers one element past an aligned address:
    "dbdc" shifts dB and dC (the adjoint scans still write du in 4-step route blocks, while the
    dB / dC partial sums keep the row layout that the element-by-element reduction reads); "gate"
    shifts dout, z and dz (the gate backward then leaves the one-workgroup-per-plane kernel for
    the tiled one, element by element).  Every gradient equals, bit for bit, that of the same call
    on aligned buffers, and nothing around the shifted outputs is written."""
    batch, H, W, dim, N = 2, 8, 12, 9, 16
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, dtype, has_z=True, seed_base=2500, with_dout=True)
    t = dict(x=to_dev(inp["x"], dtype), delta=to_dev(inp["delta"], dtype), A=to_dev(inp["A"], "f32"),
             B=to_dev(inp["B"], dtype), C=to_dev(inp["C"], dtype), D=to_dev(inp["D"], "f32"),
             delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dtype))
    dout = to_dev(inp["dout"], dtype)
    ref = ss.ss2d_bwd(**t, dout=dout)
    tdt = t["x"].dtype

    def shifted_out(like):  # an output one element past an aligned address, with guard bands
        n = like.numel()
        gd = Guarded((n + 1,), like.dtype, init=torch.zeros(n + 1, dtype=like.dtype))
        return gd, gd.t[1:].view(like.shape)

    guards = []
    z_in, dout_in = t["z"], dout
    if shift == "dbdc":
        gB, dB = shifted_out(t["B"])
        gC, dC = shifted_out(t["C"])
        guards += [gB, gC]
        dz = torch.empty_like(t["x"])
    else:
        dB, dC = torch.empty_like(t["B"]), torch.empty_like(t["C"])
        gz, dz = shifted_out(t["x"])
        guards.append(gz)
        z_in, dout_in = _shifted_copy(t["z"]), _shifted_copy(dout)
    dx = torch.empty_like(t["x"])
    ddelta = torch.empty_like(t["delta"])
    dA, dD, dbias = torch.empty_like(t["A"]), torch.empty_like(t["D"]), torch.empty_like(t["delta_bias"])
    nbytes = ss.ss2d_workspace_bytes(batch, dim, H, W, N, tdt)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a = bnd.SS2DBwdArgs(x=_p(t["x"]), delta=_p(t["delta"]), A=_p(t["A"]), Bm=_p(t["B"]), Cm=_p(t["C"]),
                        Dskip=_p(t["D"]), delta_bias=_p(t["delta_bias"]), z=_p(z_in), dout=_p(dout_in), dx=_p(dx),
                        ddelta=_p(ddelta), dA=_p(dA), dBm=_p(dB), dCm=_p(dC), dDskip=_p(dD), ddelta_bias=_p(dbias),
                        dz=_p(dz), workspace=_p(ws), workspace_bytes=nbytes, batch=batch, dim=dim, height=H, width=W,
                        dstate=N, dtype=_dt(t["x"]), delta_softplus=1, workspace_has_states=0, conv_k=0,
                        layer_norm=0, ln_eps=1e-5, dt_rank=0)
    assert bnd.lib().ss2d_bwd(ctypes.byref(a), _stream()) == 0
    torch.cuda.synchronize()
    for gd in guards:
        assert gd.intact()
        assert float(gd.t[0]) == 0.0
    got = {"dx": dx, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "ddelta_bias": dbias, "dz": dz}
    for k, v in got.items():
        assert torch.equal(v, ref[k]), k


@pytest.mark.parametrize("case", [(2, 197, 40, 16, "bf16"), (1, 1024, 16, 16, "f32"), (3, 31, 9, 4, "bf16")], ids=str)
def test_guard_vim_bidir(case):
    batch, L, dim, N, dtype = case
    inp = synth.make_vim_inputs(batch, L, dim, N, dtype, has_z=True, seed_base=2300 + L, with_dout=True)
    t = {k: to_dev(inp[k], dtype) for k in ("u", "delta", "B", "C", "z", "dout")}
    t.update(A=to_dev(inp["A"], "f32"), D=to_dev(inp["D"], "f32"), delta_bias=to_dev(inp["delta_bias"], "f32"))
    kw = dict(D=t["D"], delta_bias=t["delta_bias"], z=t["z"])
    ref_out = ss.vim_bidir_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], **kw)
    ref_g = ss.vim_bidir_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], **kw, dout=t["dout"])
    nbytes = ss.vim_bidir_workspace_bytes(batch, dim, L, N, t["u"].dtype)
    common = dict(u=_p(t["u"]), delta=_p(t["delta"]), A=_p(t["A"]), Bm=_p(t["B"]), Cm=_p(t["C"]), Dskip=_p(t["D"]),
                  delta_bias=_p(t["delta_bias"]), z=_p(t["z"]), workspace_bytes=nbytes, batch=batch, dim=dim,
                  seqlen=L, dstate=N, dtype=_dt(t["u"]), delta_softplus=1)
    out, ws = Guarded(t["z"].shape, t["u"].dtype), Guarded((nbytes,), torch.uint8)
    a = bnd.VimFwdArgs(**common, out=out.ptr, workspace=ws.ptr, keep_states=0)
    assert bnd.lib().vim_bidir_fwd(ctypes.byref(a), _stream()) == 0
    _check_all({"out": out, "workspace": ws}, {"out": ref_out})
    g = {"du": Guarded(t["u"].shape, t["u"].dtype), "ddelta": Guarded(t["u"].shape, t["u"].dtype),
         "dB": Guarded(t["B"].shape, t["u"].dtype), "dC": Guarded(t["C"].shape, t["u"].dtype),
         "dz": Guarded(t["z"].shape, t["u"].dtype), "dA": Guarded(t["A"].shape, torch.float32),
         "dD": Guarded(t["D"].shape, torch.float32), "ddelta_bias": Guarded(t["D"].shape, torch.float32),
         "workspace": Guarded((nbytes,), torch.uint8)}
    b = bnd.VimBwdArgs(**common, dout=_p(t["dout"]), du=g["du"].ptr, ddelta=g["ddelta"].ptr, dA=g["dA"].ptr,
                       dBm=g["dB"].ptr, dCm=g["dC"].ptr, dDskip=g["dD"].ptr, ddelta_bias=g["ddelta_bias"].ptr,
                       dz=g["dz"].ptr, workspace=g["workspace"].ptr, workspace_has_states=0)
    assert bnd.lib().vim_bidir_bwd(ctypes.byref(b), _stream()) == 0
    _check_all(g, ref_g)


@pytest.mark.parametrize("case", [(3, 38, 16, 2, "bf16"), (2, 5, 3, 1, "f32")], ids=str)
def test_guard_selective_scan_step(case):
    batch, dim, N, G, dtype = case
    inp = synth.make_ss_inputs(batch, dim, N, 1, G, dtype, has_z=True, seed_base=2400 + dim)
    x, delta, z = (to_dev(inp[k][..., 0].copy(), dtype) for k in ("u", "delta", "z"))
    Bm, Cm = (to_dev(inp[k][..., 0].copy(), dtype) for k in ("B", "C"))
    A, D, bias = to_dev(inp["A"], "f32"), to_dev(inp["D"], "f32"), to_dev(inp["delta_bias"], "f32")
    s0 = torch.randn(batch, dim, N, device="cuda")
    ref_state = s0.clone()
    ref_out = ss.selective_scan_step(ref_state, x, delta, A, Bm, Cm, D=D, z=z, delta_bias=bias, delta_softplus=True)
    state, out = Guarded((batch, dim, N), torch.float32, init=s0), Guarded((batch, dim), x.dtype)
    a = bnd.SsStepArgs(state=state.ptr, x=_p(x), delta=_p(delta), A=_p(A), Bm=_p(Bm), Cm=_p(Cm), Dskip=_p(D), z=_p(z),
                       delta_bias=_p(bias), out=out.ptr, batch=batch, dim=dim, dstate=N, ngroups=G,
                       dtype=_dt(x), delta_softplus=1)
    assert bnd.lib().selective_scan_step(ctypes.byref(a), _stream()) == 0
    _check_all({"state": state, "out": out}, {"state": ref_state, "out": ref_out})


# ----------------------------------------------------------------------------------------------
def _classes(a):
    """0 finite, 1 NaN, 2 +Inf, 3 -Inf."""
    a = np.asarray(a)
    return np.where(np.isnan(a), 1, np.where(np.isposinf(a), 2, np.where(np.isneginf(a), 3, 0)))


@pytest.mark.parametrize("case", [(2, 7, 9, 20, 16, "f32"), (2, 8, 8, 5, 4, "f32"), (1, 12, 16, 40, 8, "bf16")],
                         ids=str)
def test_ss2d_nan_propagates(case):
    """NaN planted in the raw delta of one route at one late step, in B of another route, and in z at
    one pixel: the NaN outputs are exactly the oracle's (the routes after the planted step, every
    channel of the image for B, the one pixel for z); the rest stays finite."""
    batch, H, W, dim, N, dtype = case
    L = H * W
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, dtype, has_z=True, seed_base=2500 + L)
    ref = {k: f64(inp[k], dtype) for k in ("x", "delta", "B", "C", "z")}
    ref.update(A=inp["A"].astype(np.float64), D=inp["D"].astype(np.float64),
               delta_bias=inp["delta_bias"].astype(np.float64))
    ref["delta"][0, 0, 1, L - 3] = np.nan      # route 0, channel 1: the last three pixels of the plane
    ref["B"][batch - 1, 3, N - 1, L - 2] = np.nan  # route 3 of the last image: two steps, every channel
    ref["z"][0, dim - 1, H // 2, W // 3] = np.nan  # one pixel
    dev = {k: to_dev(synth.f32_to_bf16_bits(v.astype(np.float32)) if dtype == "bf16" else v.astype(np.float32), dtype)
           for k, v in ref.items() if k in ("x", "delta", "B", "C", "z")}
    dev.update(A=to_dev(inp["A"], "f32"), D=to_dev(inp["D"], "f32"), delta_bias=to_dev(inp["delta_bias"], "f32"))
    want = _classes(oracle.ss2d_fwd(**ref))
    assert (want == 1).any() and (want == 0).any()
    got = _classes(to_f64(ss.ss2d_fwd(**dev)))
    np.testing.assert_array_equal(got, want)
    plan = ss.SS2DForwardPlan(**dev)  # the three stages (where the call above ran one kernel per plane)
    for stage in (0, 1, 2):
        plan.run_stage(stage)
    np.testing.assert_array_equal(_classes(to_f64(plan.out)), want)


@pytest.mark.parametrize("case", [(2, 64, 16, 300, 2, "f32"), (1, 16, 8, 3000, 1, "bf16"), (2, 40, 1, 77, 1, "f32")],
                         ids=str)
def test_selective_scan_nan_inf_propagate(case):
    """A NaN in u at one step of one row and +Inf in the raw delta at one step of another: the
    output is non-finite exactly where the oracle's is, and NaN exactly where it is for the NaN row
    (with a step of infinite delta the state jumps to infinity; which of its sums come out NaN or
    +-Inf is exact in both, as no finite value is involved)."""
    batch, dim, N, L, G, dtype = case
    inp = synth.make_ss_inputs(batch, dim, N, L, G, dtype, has_z=True, seed_base=2600 + L)
    ref = {k: f64(inp[k], dtype) for k in ("u", "delta", "B", "C", "z")}
    ref.update(A=inp["A"].astype(np.float64), D=inp["D"].astype(np.float64),
               delta_bias=inp["delta_bias"].astype(np.float64))
    ref["u"][0, 1, L // 2] = np.nan
    ref["delta"][batch - 1, dim - 1, L - L // 3] = np.inf
    dev = {k: to_dev(synth.f32_to_bf16_bits(v.astype(np.float32)) if dtype == "bf16" else v.astype(np.float32), dtype)
           for k, v in ref.items() if k in ("u", "delta", "B", "C", "z")}
    dev.update(A=to_dev(inp["A"], "f32"), D=to_dev(inp["D"], "f32"), delta_bias=to_dev(inp["delta_bias"], "f32"))
    want = _classes(oracle.ss_fwd(**ref, delta_softplus=True))
    got = _classes(to_f64(ss.selective_scan_fwd(**dev, delta_softplus=True)))
    np.testing.assert_array_equal(got != 0, want != 0)
    np.testing.assert_array_equal(got[0, 1], want[0, 1])
    assert (want != 0).sum() < want.size // 2


def test_ss2d_bwd_nan_propagates():
    """A NaN in dout at one pixel: the non-finite gradients are exactly the oracle's."""
    batch, H, W, dim, N = 2, 7, 9, 12, 8
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, "f32", has_z=True, seed_base=2700, with_dout=True)
    ref = {k: inp[k].astype(np.float64) for k in ("x", "delta", "A", "B", "C", "D", "delta_bias", "z")}
    dout = inp["dout"].copy()
    dout[1, 3, 2, 5] = np.nan
    dev = {k: to_dev(inp[k], "f32") for k in ("x", "delta", "A", "B", "C", "D", "delta_bias", "z")}
    g = ss.ss2d_bwd(**dev, dout=to_dev(dout, "f32"))
    r = oracle.ss2d_bwd(**ref, dout=dout.astype(np.float64))
    for k in ("dx", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz"):
        want = _classes(r[k])
        np.testing.assert_array_equal(_classes(to_f64(g[k])) != 0, want != 0, err_msg=k)


# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_equals_unchunked_ss2d(dtype):
    """Stage-1 shapes (56x56, D=192, N=16): one image alone (98 chunks of 32 steps per route row,
    joined by the pair operator) against the same image inside a 64-image launch (every row run
    whole), forward and backward, image for image."""
    H = W = 56
    dim, N, nb = 192, 16, 64
    inp = synth.make_ss2d_inputs(nb, H, W, dim, N, dtype, has_z=True, seed_base=2800, with_dout=True)
    full = {k: to_dev(inp[k], dtype) for k in ("x", "delta", "B", "C", "z", "dout")}
    full.update(A=to_dev(inp["A"], "f32"), D=to_dev(inp["D"], "f32"), delta_bias=to_dev(inp["delta_bias"], "f32"))
    one = {k: (v[:1].contiguous() if k in ("x", "delta", "B", "C", "z", "dout") else v) for k, v in full.items()}
    args = lambda t: {k: v for k, v in t.items() if k != "dout"}
    out_full = ss.ss2d_fwd(**args(full))
    out_one = ss.ss2d_fwd(**args(one))
    tol = 1e-5 if dtype == "f32" else 8e-3  # bf16: at most one rounding step of the output apart
    assert rel_err(to_f64(out_one), to_f64(out_full[:1])) <= tol
    g_full = ss.ss2d_bwd(**args(full), dout=full["dout"])
    g_one = ss.ss2d_bwd(**args(one), dout=one["dout"])
    for k in ("dx", "ddelta", "dB", "dC", "dz"):
        assert rel_err(to_f64(g_one[k]), to_f64(g_full[k][:1])) <= (1e-4 if dtype == "f32" else 8e-3), k


def test_chunked_equals_unchunked_selective_scan():
    """The generic scan: 2 rows of 4096 steps (chunked) against the same rows among 1600 copies
    (enough rows to fill the GPU, so every row runs whole)."""
    dim, N, L = 2, 16, 4096
    inp = synth.make_ss_inputs(1, dim, N, L, 1, "f32", has_z=True, seed_base=2900, with_dout=True)
    t = {k: to_dev(inp[k], "f32") for k in ("u", "delta", "B", "C", "z", "dout")}
    A, D, bias = to_dev(inp["A"], "f32"), to_dev(inp["D"], "f32"), to_dev(inp["delta_bias"], "f32")
    rep = 1600
    big = {k: t[k].repeat(rep, 1, 1) if t[k].dim() == 3 else t[k].repeat(rep, 1, 1, 1) for k in t}
    o1, s1 = ss.selective_scan_fwd(t["u"], t["delta"], A, t["B"], t["C"], D=D, z=t["z"], delta_bias=bias,
                                   delta_softplus=True, return_last_state=True)
    o2, s2 = ss.selective_scan_fwd(big["u"], big["delta"], A, big["B"], big["C"], D=D, z=big["z"], delta_bias=bias,
                                   delta_softplus=True, return_last_state=True)
    assert rel_err(to_f64(o1), to_f64(o2[:1])) <= 1e-5
    assert rel_err(to_f64(s1), to_f64(s2[:1])) <= 1e-5
    g1 = ss.selective_scan_bwd(t["u"], t["delta"], A, t["B"], t["C"], D=D, z=t["z"], delta_bias=bias,
                               dout=t["dout"], delta_softplus=True)
    g2 = ss.selective_scan_bwd(big["u"], big["delta"], A, big["B"], big["C"], D=D, z=big["z"], delta_bias=bias,
                               dout=big["dout"], delta_softplus=True)
    for k in ("du", "ddelta", "dB", "dC", "dz"):
        assert rel_err(to_f64(g1[k]), to_f64(g2[k][:1])) <= 1e-4, k
    for k in ("dA", "dD", "ddelta_bias"):  # the big launch sums 1600 identical images
        assert rel_err(to_f64(g1[k]) * rep, to_f64(g2[k])) <= 1e-4, k
