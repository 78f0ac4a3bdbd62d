"""ctypes binding of libss2d.so (include/ss2d.h).  Argument marshalling only.

Each function here has the name of the C entry point it calls, takes torch tensors that
already live on a ROCm device, allocates the outputs (and, when not given, the workspace)
with torch, and enqueues the library call on torch's current stream of that device.  Every
step of the computation runs in the library's HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libss2d.so")

SS2D_OK, SS2D_ERR_INVALID_ARGUMENT, SS2D_ERR_UNSUPPORTED, SS2D_ERR_HIP, SS2D_ERR_TOO_LARGE = 0, 1, 2, 3, 4
DTYPE_F32, DTYPE_BF16 = 0, 1
ABI_VERSION = 8

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t


class SsFwdArgs(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("u", "delta", "A", "Bm", "Cm", "Dskip", "z", "delta_bias", "out",
                                  "last_state", "workspace")] + [
        ("workspace_bytes", _sz), ("batch", _i64), ("dim", _i64), ("dstate", _i64), ("seqlen", _i64),
        ("ngroups", _i64), ("dtype", _int), ("delta_softplus", _int)]


class SsBwdArgs(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("u", "delta", "A", "Bm", "Cm", "Dskip", "z", "delta_bias", "dout", "du",
                                  "ddelta", "dA", "dBm", "dCm", "dDskip", "dz", "ddelta_bias", "workspace")] + [
        ("workspace_bytes", _sz), ("workspace_has_states", _int), ("batch", _i64), ("dim", _i64),
        ("dstate", _i64), ("seqlen", _i64), ("ngroups", _i64), ("dtype", _int), ("delta_softplus", _int)]


class SS2DFwdArgs(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("x", "delta", "A", "Bm", "Cm", "Dskip", "delta_bias", "z", "out",
                                  "workspace")] + [
        ("workspace_bytes", _sz), ("batch", _i64), ("dim", _i64), ("height", _i64), ("width", _i64),
        ("dstate", _i64), ("dtype", _int), ("delta_softplus", _int), ("keep_states", _int),
        ("conv_w", _p), ("conv_b", _p), ("conv_k", _int),
        ("layer_norm", _int), ("ln_w", _p), ("ln_b", _p), ("ln_eps", ctypes.c_float),
        ("x_proj_w", _p), ("dt_proj_w", _p), ("dt_rank", _int)]


class SS2DBwdArgs(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("x", "delta", "A", "Bm", "Cm", "Dskip", "delta_bias", "z", "dout", "dx",
                                  "ddelta", "dA", "dBm", "dCm", "dDskip", "ddelta_bias", "dz", "workspace")] + [
        ("workspace_bytes", _sz), ("batch", _i64), ("dim", _i64), ("height", _i64), ("width", _i64),
        ("dstate", _i64), ("dtype", _int), ("delta_softplus", _int), ("workspace_has_states", _int),
        ("conv_w", _p), ("conv_b", _p), ("conv_k", _int), ("dconv_w", _p), ("dconv_b", _p),
        ("layer_norm", _int), ("ln_w", _p), ("ln_b", _p), ("ln_eps", ctypes.c_float), ("dln_w", _p), ("dln_b", _p),
        ("x_proj_w", _p), ("dt_proj_w", _p), ("dt_rank", _int), ("dx_proj_w", _p), ("ddt_proj_w", _p)]


class SsStepArgs(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("state", "x", "delta", "A", "Bm", "Cm", "Dskip", "z", "delta_bias", "out")] + [
        ("batch", _i64), ("dim", _i64), ("dstate", _i64), ("ngroups", _i64), ("dtype", _int),
        ("delta_softplus", _int)]


class VimFwdArgs(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("u", "delta", "A", "Bm", "Cm", "Dskip", "delta_bias", "z", "out",
                                  "workspace")] + [
        ("workspace_bytes", _sz), ("batch", _i64), ("dim", _i64), ("seqlen", _i64), ("dstate", _i64),
        ("dtype", _int), ("delta_softplus", _int), ("keep_states", _int)]


class VimBwdArgs(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("u", "delta", "A", "Bm", "Cm", "Dskip", "delta_bias", "z", "dout", "du",
                                  "ddelta", "dA", "dBm", "dCm", "dDskip", "ddelta_bias", "dz", "workspace")] + [
        ("workspace_bytes", _sz), ("batch", _i64), ("dim", _i64), ("seqlen", _i64), ("dstate", _i64),
        ("dtype", _int), ("delta_softplus", _int), ("workspace_has_states", _int)]


_lib = None


def lib():
    """Load libss2d.so (built by __graft_entry__.build()); fail loudly if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        L.ss2d_abi_version.restype = _int
        L.ss2d_abi_version.argtypes = []
        L.ss2d_status_string.restype = ctypes.c_char_p
        L.ss2d_status_string.argtypes = [_int]
        for name in ("ss2d_cross_scan", "ss2d_cross_merge"):
            f = getattr(L, name)
            f.restype = _int
            f.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _int, _p]
        L.selective_scan_workspace_bytes.restype = _sz
        L.selective_scan_workspace_bytes.argtypes = [_i64] * 5
        L.ss2d_workspace_bytes.restype = _sz
        L.ss2d_workspace_bytes.argtypes = [_i64] * 5 + [_int]
        L.ss2d_proj_workspace_bytes.restype = _sz
        L.ss2d_proj_workspace_bytes.argtypes = [_i64] * 6 + [_int]
        L.ss2d_fwd_stage.restype = _int
        L.ss2d_fwd_stage.argtypes = [ctypes.POINTER(SS2DFwdArgs), _int, _p]
        L.ss2d_fwd_single_kernel.restype = _int
        L.ss2d_fwd_single_kernel.argtypes = [ctypes.POINTER(SS2DFwdArgs)]
        L.vim_bidir_workspace_bytes.restype = _sz
        L.vim_bidir_workspace_bytes.argtypes = [_i64] * 4 + [_int]
        L.vim_bidir_fwd_stage.restype = _int
        L.vim_bidir_fwd_stage.argtypes = [ctypes.POINTER(VimFwdArgs), _int, _p]
        L.ss2d_fwd_noalloc_max_workspace_bytes.restype = _sz
        L.ss2d_fwd_noalloc_max_workspace_bytes.argtypes = []
        for name, st in (("selective_scan_fwd", SsFwdArgs), ("selective_scan_bwd", SsBwdArgs),
                         ("ss2d_fwd", SS2DFwdArgs), ("ss2d_fwd_noalloc", SS2DFwdArgs), ("ss2d_bwd", SS2DBwdArgs),
                         ("vim_bidir_fwd", VimFwdArgs), ("vim_bidir_bwd", VimBwdArgs),
                         ("selective_scan_step", SsStepArgs)):
            f = getattr(L, name)
            f.restype = _int
            f.argtypes = [ctypes.POINTER(st), _p]
        if L.ss2d_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libss2d ABI {L.ss2d_abi_version()} != binding ABI {ABI_VERSION}")
        _lib = L
    return _lib


class SS2DError(RuntimeError):
    pass


def _check(status: int, what: str):
    if status != SS2D_OK:
        raise SS2DError(f"{what}: {lib().ss2d_status_string(status).decode()} (status {status})")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return DTYPE_F32
    if t == torch.bfloat16:
        return DTYPE_BF16
    raise SS2DError(f"unsupported I/O dtype {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor) -> torch.device:
    if not t.is_cuda:
        raise SS2DError("tensors must live on a ROCm device")
    return t.device


def _c(t, dtype=None):
    """Contiguous (as the pages' wrapper does for every input), optionally cast (fp32 params)."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        t = t.to(dtype)
    return t.contiguous()


def _workspace(nbytes: int, device, workspace=None):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise SS2DError("workspace too small")
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------------------
def ss2d_cross_scan(x: torch.Tensor) -> torch.Tensor:
    x = _c(x)
    B, C, H, W = x.shape
    xs = torch.empty((B, 4, C, H * W), dtype=x.dtype, device=_dev(x))
    _check(lib().ss2d_cross_scan(_ptr(x), _ptr(xs), B, C, H, W, _dtype_code(x.dtype), _stream(x.device)),
           "ss2d_cross_scan")
    return xs


def ss2d_cross_merge(ys: torch.Tensor, height: int, width: int) -> torch.Tensor:
    ys = _c(ys)
    B, K, C, L = ys.shape
    if K != 4 or L != height * width:
        raise SS2DError("ys must be (batch, 4, channels, height*width)")
    y = torch.empty((B, C, height, width), dtype=ys.dtype, device=_dev(ys))
    _check(lib().ss2d_cross_merge(_ptr(ys), _ptr(y), B, C, height, width, _dtype_code(ys.dtype),
                                  _stream(ys.device)), "ss2d_cross_merge")
    return y


def selective_scan_workspace_bytes(batch, dim, dstate, seqlen, ngroups) -> int:
    return int(lib().selective_scan_workspace_bytes(batch, dim, dstate, seqlen, ngroups))


def ss2d_workspace_bytes(batch, dim, height, width, dstate, dtype: torch.dtype, dt_rank: int = 0) -> int:
    """Workspace of ss2d_fwd / ss2d_bwd; with dt_rank > 0, of the path with the Δ/B/C producer."""
    if dt_rank:
        return int(lib().ss2d_proj_workspace_bytes(batch, dim, height, width, dstate, dt_rank, _dtype_code(dtype)))
    return int(lib().ss2d_workspace_bytes(batch, dim, height, width, dstate, _dtype_code(dtype)))


def _proj(x_proj_w, dt_proj_w, dim):
    """(x_proj_w, dt_proj_w, dt_rank, dstate from x_proj_w) of the Δ/B/C producer, or Nones."""
    if x_proj_w is None and dt_proj_w is None:
        return None, None, 0
    if x_proj_w is None or dt_proj_w is None:
        raise ValueError("x_proj_w and dt_proj_w go together")
    x_proj_w, dt_proj_w = _c(x_proj_w, torch.float32), _c(dt_proj_w, torch.float32)
    R = int(dt_proj_w.shape[-1])
    if tuple(dt_proj_w.shape) != (4, dim, R) or x_proj_w.dim() != 3 or x_proj_w.shape[0] != 4 or \
            x_proj_w.shape[2] != dim or (x_proj_w.shape[1] - R) % 2:
        raise ValueError(f"x_proj_w (4, R + 2N, dim) and dt_proj_w (4, dim, R) expected, got "
                         f"{tuple(x_proj_w.shape)}, {tuple(dt_proj_w.shape)}")
    return x_proj_w, dt_proj_w, R


def _bc4(Bm):
    return Bm.unsqueeze(1) if Bm.dim() == 3 else Bm  # (batch, N, L) is read as one group


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                       return_last_state=False, workspace=None):
    """Forward of the selective scan (`selective_scan_fn` shapes).  Returns out, and
    last_state when asked.  A caller-provided `workspace` (uint8 tensor of at least
    selective_scan_workspace_bytes) keeps the checkpoint states that selective_scan_bwd can
    reuse (workspace_has_states=True); without one a temporary workspace is allocated."""
    u, delta = _c(u), _c(delta)
    dev = _dev(u)
    B, C = _c(_bc4(B)), _c(_bc4(C))
    A = _c(A, torch.float32)
    D = _c(D, torch.float32)
    delta_bias = _c(delta_bias, torch.float32)
    z = _c(z)
    batch, dim, L = u.shape
    N = A.shape[1]
    G = B.shape[1]
    out = torch.empty_like(u)
    last = torch.empty((batch, dim, N), dtype=torch.float32, device=dev) if return_last_state else None
    ws = _workspace(selective_scan_workspace_bytes(batch, dim, N, L, G), dev, workspace)
    a = SsFwdArgs(u=_ptr(u), delta=_ptr(delta), A=_ptr(A), Bm=_ptr(B), Cm=_ptr(C), Dskip=_ptr(D), z=_ptr(z),
                  delta_bias=_ptr(delta_bias), out=_ptr(out), last_state=_ptr(last), workspace=_ptr(ws),
                  workspace_bytes=ws.numel() * ws.element_size(),
                  batch=batch, dim=dim, dstate=N, seqlen=L, ngroups=G, dtype=_dtype_code(u.dtype),
                  delta_softplus=int(bool(delta_softplus)))
    _check(lib().selective_scan_fwd(ctypes.byref(a), _stream(dev)), "selective_scan_fwd")
    return (out, last) if return_last_state else out


def selective_scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, dout=None, delta_softplus=False,
                       workspace=None, workspace_has_states=False):
    """Backward of selective_scan_fwd.  Returns a dict of gradients (None for absent inputs)."""
    u, delta, dout = _c(u), _c(delta), _c(dout)
    dev = _dev(u)
    squeeze = B.dim() == 3
    B, C = _c(_bc4(B)), _c(_bc4(C))
    A = _c(A, torch.float32)
    D = _c(D, torch.float32)
    delta_bias = _c(delta_bias, torch.float32)
    z = _c(z)
    batch, dim, L = u.shape
    N = A.shape[1]
    G = B.shape[1]
    du, ddelta = torch.empty_like(u), torch.empty_like(u)
    dA = torch.empty((dim, N), dtype=torch.float32, device=dev)
    dB, dC = torch.empty_like(B), torch.empty_like(C)
    dD = torch.empty(dim, dtype=torch.float32, device=dev) if D is not None else None
    dz = torch.empty_like(u) if z is not None else None
    dbias = torch.empty(dim, dtype=torch.float32, device=dev) if delta_bias is not None else None
    ws = _workspace(selective_scan_workspace_bytes(batch, dim, N, L, G), dev, workspace)
    a = SsBwdArgs(u=_ptr(u), delta=_ptr(delta), A=_ptr(A), Bm=_ptr(B), Cm=_ptr(C), Dskip=_ptr(D), z=_ptr(z),
                  delta_bias=_ptr(delta_bias), dout=_ptr(dout), du=_ptr(du), ddelta=_ptr(ddelta), dA=_ptr(dA),
                  dBm=_ptr(dB), dCm=_ptr(dC), dDskip=_ptr(dD), dz=_ptr(dz), ddelta_bias=_ptr(dbias),
                  workspace=_ptr(ws), workspace_bytes=ws.numel() * ws.element_size(),
                  workspace_has_states=int(bool(workspace_has_states)), batch=batch, dim=dim, dstate=N,
                  seqlen=L, ngroups=G, dtype=_dtype_code(u.dtype), delta_softplus=int(bool(delta_softplus)))
    _check(lib().selective_scan_bwd(ctypes.byref(a), _stream(dev)), "selective_scan_bwd")
    if squeeze:
        dB, dC = dB[:, 0], dC[:, 0]
    return {"du": du, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "dz": dz, "ddelta_bias": dbias}


def _conv_k(conv_w, dim):
    """Filter size of a depthwise filter given as (dim, k, k) or (dim, 1, k, k)."""
    if conv_w is None:
        return 0
    k = int(conv_w.shape[-1])
    if conv_w.dim() < 2 or conv_w.shape[-2] != k or conv_w.numel() != dim * k * k:
        raise ValueError(f"conv_w must be (dim, k, k) for dim={dim}, got {tuple(conv_w.shape)}")
    return k


def _ln_on(layer_norm, ln_w, ln_b):
    return int(bool(layer_norm) or ln_w is not None or ln_b is not None)


def ss2d_fwd(x, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True, workspace=None,
             out=None, keep_states=False, conv_w=None, conv_b=None, layer_norm=False, ln_w=None, ln_b=None,
             ln_eps=1e-5, x_proj_w=None, dt_proj_w=None):
    """Fused SS2D forward.  x, z: (batch, dim, H, W); delta: (batch, 4, dim, H*W);
    A: (4, dim, N) fp32; B, C: (batch, 4, N, H*W); D, delta_bias: (4, dim) fp32.  With
    keep_states the given workspace keeps what ss2d_bwd(..., workspace_has_states=True) needs.
    conv_w (dim, k, k) and conv_b (dim,), fp32, add the input front: the routes scan
    silu(depthwise_conv(x) + conv_b) instead of x.  layer_norm (implied by ln_w or ln_b, fp32
    (dim,)) adds the back half: out = LayerNorm_channels(merged) * silu(z).  x_proj_w
    (4, R + 2N, dim) and dt_proj_w (4, dim, R), fp32, add the Δ/B/C producer: delta, B and C
    (pass None) come from each route's projections of its scanned sequence."""
    x, delta = _c(x), _c(delta)
    dev = _dev(x)
    B, C, z = _c(B), _c(C), _c(z)
    A = _c(A, torch.float32)
    D = _c(D, torch.float32)
    delta_bias = _c(delta_bias, torch.float32)
    conv_w, conv_b = _c(conv_w, torch.float32), _c(conv_b, torch.float32)
    ln_w, ln_b = _c(ln_w, torch.float32), _c(ln_b, torch.float32)
    batch, dim, H, W = x.shape
    N = A.shape[-1]
    x_proj_w, dt_proj_w, R = _proj(x_proj_w, dt_proj_w, dim)
    if R and x_proj_w.shape[1] != R + 2 * N:
        raise ValueError(f"x_proj_w has {x_proj_w.shape[1]} rows, expected dt_rank + 2 dstate = {R + 2 * N}")
    if out is None:
        out = torch.empty_like(x)
    ws = _workspace(ss2d_workspace_bytes(batch, dim, H, W, N, x.dtype, R), dev, workspace)
    a = SS2DFwdArgs(x=_ptr(x), delta=_ptr(delta), A=_ptr(A), Bm=_ptr(B), Cm=_ptr(C), Dskip=_ptr(D),
                    delta_bias=_ptr(delta_bias), z=_ptr(z), out=_ptr(out), workspace=_ptr(ws),
                    workspace_bytes=ws.numel() * ws.element_size(), batch=batch, dim=dim, height=H, width=W,
                    dstate=N, dtype=_dtype_code(x.dtype), delta_softplus=int(bool(delta_softplus)),
                    keep_states=int(bool(keep_states)), conv_w=_ptr(conv_w), conv_b=_ptr(conv_b),
                    conv_k=_conv_k(conv_w, dim), layer_norm=_ln_on(layer_norm, ln_w, ln_b), ln_w=_ptr(ln_w),
                    ln_b=_ptr(ln_b), ln_eps=float(ln_eps), x_proj_w=_ptr(x_proj_w), dt_proj_w=_ptr(dt_proj_w),
                    dt_rank=R)
    _check(lib().ss2d_fwd(ctypes.byref(a), _stream(dev)), "ss2d_fwd")
    return out


def ss2d_fwd_noalloc_max_workspace_bytes() -> int:
    return int(lib().ss2d_fwd_noalloc_max_workspace_bytes())


def ss2d_fwd_noalloc(x, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True, out=None,
                     conv_w=None, conv_b=None, layer_norm=False, ln_w=None, ln_b=None, ln_eps=1e-5, x_proj_w=None,
                     dt_proj_w=None):
    """ss2d_fwd without a workspace: the library's fixed per-GPU scratch serves instead (calls
    that may overlap in time on one GPU race on it).  With `out` given and contiguous inputs of
    the right types, nothing is allocated.  Raises SS2DError (status SS2D_ERR_TOO_LARGE) when the
    call needs more scratch than ss2d_fwd_noalloc_max_workspace_bytes()."""
    x, delta = _c(x), _c(delta)
    dev = _dev(x)
    B, C, z = _c(B), _c(C), _c(z)
    A = _c(A, torch.float32)
    D = _c(D, torch.float32)
    delta_bias = _c(delta_bias, torch.float32)
    conv_w, conv_b = _c(conv_w, torch.float32), _c(conv_b, torch.float32)
    ln_w, ln_b = _c(ln_w, torch.float32), _c(ln_b, torch.float32)
    batch, dim, H, W = x.shape
    N = A.shape[-1]
    x_proj_w, dt_proj_w, R = _proj(x_proj_w, dt_proj_w, dim)
    if out is None:
        out = torch.empty_like(x)
    a = SS2DFwdArgs(x=_ptr(x), delta=_ptr(delta), A=_ptr(A), Bm=_ptr(B), Cm=_ptr(C), Dskip=_ptr(D),
                    delta_bias=_ptr(delta_bias), z=_ptr(z), out=_ptr(out), workspace=None, workspace_bytes=0,
                    batch=batch, dim=dim, height=H, width=W, dstate=N, dtype=_dtype_code(x.dtype),
                    delta_softplus=int(bool(delta_softplus)), keep_states=0, conv_w=_ptr(conv_w), conv_b=_ptr(conv_b),
                    conv_k=_conv_k(conv_w, dim), layer_norm=_ln_on(layer_norm, ln_w, ln_b), ln_w=_ptr(ln_w),
                    ln_b=_ptr(ln_b), ln_eps=float(ln_eps), x_proj_w=_ptr(x_proj_w), dt_proj_w=_ptr(dt_proj_w),
                    dt_rank=R)
    _check(lib().ss2d_fwd_noalloc(ctypes.byref(a), _stream(dev)), "ss2d_fwd_noalloc")
    return out


class SS2DForwardPlan:
    """A prepared ss2d_fwd call: argument block, workspace and output kept alive, so that
    repeated launches (benchmarks, stage timing) cost one ctypes call each."""

    def __init__(self, x, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True, workspace=None,
                 out=None, keep_states=False, conv_w=None, conv_b=None, layer_norm=False, ln_w=None, ln_b=None,
                 ln_eps=1e-5, x_proj_w=None, dt_proj_w=None):
        x, delta = _c(x), _c(delta)
        self.device = _dev(x)
        B, C, z = _c(B), _c(C), _c(z)
        A = _c(A, torch.float32)
        D = _c(D, torch.float32)
        delta_bias = _c(delta_bias, torch.float32)
        conv_w, conv_b = _c(conv_w, torch.float32), _c(conv_b, torch.float32)
        ln_w, ln_b = _c(ln_w, torch.float32), _c(ln_b, torch.float32)
        batch, dim, H, W = x.shape
        N = A.shape[-1]
        x_proj_w, dt_proj_w, R = _proj(x_proj_w, dt_proj_w, dim)
        self.out = torch.empty_like(x) if out is None else out
        self.workspace = _workspace(ss2d_workspace_bytes(batch, dim, H, W, N, x.dtype, R), self.device, workspace)
        self._keep = (x, delta, A, B, C, D, delta_bias, z, conv_w, conv_b, ln_w, ln_b, x_proj_w, dt_proj_w)
        self.args = SS2DFwdArgs(x=_ptr(x), delta=_ptr(delta), A=_ptr(A), Bm=_ptr(B), Cm=_ptr(C), Dskip=_ptr(D),
                                delta_bias=_ptr(delta_bias), z=_ptr(z), out=_ptr(self.out),
                                workspace=_ptr(self.workspace),
                                workspace_bytes=self.workspace.numel() * self.workspace.element_size(),
                                batch=batch, dim=dim, height=H, width=W, dstate=N, dtype=_dtype_code(x.dtype),
                                delta_softplus=int(bool(delta_softplus)), keep_states=int(bool(keep_states)),
                                conv_w=_ptr(conv_w), conv_b=_ptr(conv_b), conv_k=_conv_k(conv_w, dim),
                                layer_norm=_ln_on(layer_norm, ln_w, ln_b), ln_w=_ptr(ln_w), ln_b=_ptr(ln_b),
                                ln_eps=float(ln_eps), x_proj_w=_ptr(x_proj_w), dt_proj_w=_ptr(dt_proj_w),
                                dt_rank=R)

    @property
    def single_kernel(self) -> bool:
        """Whether run() launches one kernel per plane (ss2d_fwd_single_kernel) instead of the
        three stages of run_stage."""
        return bool(lib().ss2d_fwd_single_kernel(ctypes.byref(self.args)))

    def run(self):
        _check(lib().ss2d_fwd(ctypes.byref(self.args), _stream(self.device)), "ss2d_fwd")
        return self.out

    def run_stage(self, stage: int):
        _check(lib().ss2d_fwd_stage(ctypes.byref(self.args), int(stage), _stream(self.device)), "ss2d_fwd_stage")
        return self.out


def ss2d_bwd(x, delta, A, B, C, D=None, delta_bias=None, z=None, dout=None, delta_softplus=True,
             workspace=None, workspace_has_states=False, conv_w=None, conv_b=None, layer_norm=False, ln_w=None,
             ln_b=None, ln_eps=1e-5, x_proj_w=None, dt_proj_w=None):
    """Backward of ss2d_fwd; returns a dict of gradients (None for absent inputs).  With
    workspace_has_states, `workspace` must be the one a forward with keep_states=True used for
    the same inputs (the forward is then not recomputed).  With the input front (conv_w,
    conv_b) dx is the gradient w.r.t. the convolution's input and the dict also holds
    dconv_w and dconv_b; with the LayerNorm it holds dln_w and dln_b; with the Δ/B/C producer it
    holds dx_proj_w and ddt_proj_w (and ddelta, dB, dC are None: delta, B, C are internal)."""
    x, delta, dout = _c(x), _c(delta), _c(dout)
    dev = _dev(x)
    B, C, z = _c(B), _c(C), _c(z)
    A = _c(A, torch.float32)
    D = _c(D, torch.float32)
    delta_bias = _c(delta_bias, torch.float32)
    conv_w, conv_b = _c(conv_w, torch.float32), _c(conv_b, torch.float32)
    dconv_w = torch.empty_like(conv_w) if conv_w is not None else None
    dconv_b = torch.empty_like(conv_b) if conv_b is not None else None
    ln_w, ln_b = _c(ln_w, torch.float32), _c(ln_b, torch.float32)
    ln = _ln_on(layer_norm, ln_w, ln_b)
    dln_w = torch.empty_like(ln_w) if ln_w is not None else None
    dln_b = torch.empty_like(ln_b) if ln_b is not None else None
    batch, dim, H, W = x.shape
    N = A.shape[-1]
    x_proj_w, dt_proj_w, R = _proj(x_proj_w, dt_proj_w, dim)
    if R and x_proj_w.shape[1] != R + 2 * N:
        raise ValueError(f"x_proj_w has {x_proj_w.shape[1]} rows, expected dt_rank + 2 dstate = {R + 2 * N}")
    dx = torch.empty_like(x)
    ddelta = torch.empty_like(delta) if not R else None
    dA = torch.empty_like(A)
    dB, dC = (torch.empty_like(B), torch.empty_like(C)) if not R else (None, None)
    dD = torch.empty_like(D) if D is not None else None
    dbias = torch.empty_like(delta_bias) if delta_bias is not None else None
    dz = torch.empty_like(z) if z is not None else None
    dxp = torch.empty_like(x_proj_w) if R else None
    ddtp = torch.empty_like(dt_proj_w) if R else None
    ws = _workspace(ss2d_workspace_bytes(batch, dim, H, W, N, x.dtype, R), dev, workspace)
    a = SS2DBwdArgs(x=_ptr(x), delta=_ptr(delta), A=_ptr(A), Bm=_ptr(B), Cm=_ptr(C), Dskip=_ptr(D),
                    delta_bias=_ptr(delta_bias), z=_ptr(z), dout=_ptr(dout), dx=_ptr(dx), ddelta=_ptr(ddelta),
                    dA=_ptr(dA), dBm=_ptr(dB), dCm=_ptr(dC), dDskip=_ptr(dD), ddelta_bias=_ptr(dbias), dz=_ptr(dz),
                    workspace=_ptr(ws), workspace_bytes=ws.numel() * ws.element_size(), batch=batch, dim=dim,
                    height=H, width=W, dstate=N, dtype=_dtype_code(x.dtype),
                    delta_softplus=int(bool(delta_softplus)), workspace_has_states=int(bool(workspace_has_states)),
                    conv_w=_ptr(conv_w), conv_b=_ptr(conv_b), conv_k=_conv_k(conv_w, dim), dconv_w=_ptr(dconv_w),
                    dconv_b=_ptr(dconv_b), layer_norm=ln, ln_w=_ptr(ln_w), ln_b=_ptr(ln_b), ln_eps=float(ln_eps),
                    dln_w=_ptr(dln_w), dln_b=_ptr(dln_b), x_proj_w=_ptr(x_proj_w), dt_proj_w=_ptr(dt_proj_w),
                    dt_rank=R, dx_proj_w=_ptr(dxp), ddt_proj_w=_ptr(ddtp))
    _check(lib().ss2d_bwd(ctypes.byref(a), _stream(dev)), "ss2d_bwd")
    g = {"dx": dx, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "ddelta_bias": dbias, "dz": dz}
    if conv_w is not None:
        g.update(dconv_w=dconv_w, dconv_b=dconv_b)
    if ln:
        g.update(dln_w=dln_w, dln_b=dln_b)
    if R:
        g.update(dx_proj_w=dxp, ddt_proj_w=ddtp)
    return g


def vim_bidir_workspace_bytes(batch, dim, seqlen, dstate, dtype: torch.dtype) -> int:
    return int(lib().vim_bidir_workspace_bytes(batch, dim, seqlen, dstate, _dtype_code(dtype)))


class VimForwardPlan:
    """A prepared vim_bidir_fwd call (argument block, workspace and output kept alive).
    u, delta: (batch, 2, dim, L); A: (2, dim, N); B, C: (batch, 2, N, L); D, delta_bias: (2, dim);
    z: (batch, dim, L).  With keep_states the workspace also keeps what
    vim_bidir_bwd(..., workspace_has_states=True) needs."""

    def __init__(self, u, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True, workspace=None,
                 out=None, keep_states=False):
        u, delta = _c(u), _c(delta)
        self.device = _dev(u)
        B, C, z = _c(B), _c(C), _c(z)
        A = _c(A, torch.float32)
        D = _c(D, torch.float32)
        delta_bias = _c(delta_bias, torch.float32)
        batch, K, dim, L = u.shape
        if K != 2:
            raise SS2DError("u must be (batch, 2, dim, L)")
        N = A.shape[-1]
        self.out = torch.empty((batch, dim, L), dtype=u.dtype, device=self.device) if out is None else out
        self.workspace = _workspace(vim_bidir_workspace_bytes(batch, dim, L, N, u.dtype), self.device, workspace)
        self._keep = (u, delta, A, B, C, D, delta_bias, z)
        self.args = VimFwdArgs(u=_ptr(u), delta=_ptr(delta), A=_ptr(A), Bm=_ptr(B), Cm=_ptr(C), Dskip=_ptr(D),
                               delta_bias=_ptr(delta_bias), z=_ptr(z), out=_ptr(self.out),
                               workspace=_ptr(self.workspace),
                               workspace_bytes=self.workspace.numel() * self.workspace.element_size(),
                               batch=batch, dim=dim, seqlen=L, dstate=N, dtype=_dtype_code(u.dtype),
                               delta_softplus=int(bool(delta_softplus)), keep_states=int(bool(keep_states)))

    def run(self):
        _check(lib().vim_bidir_fwd(ctypes.byref(self.args), _stream(self.device)), "vim_bidir_fwd")
        return self.out

    def run_stage(self, stage: int):
        _check(lib().vim_bidir_fwd_stage(ctypes.byref(self.args), int(stage), _stream(self.device)),
               "vim_bidir_fwd_stage")
        return self.out


def vim_bidir_fwd(u, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True, workspace=None,
                  keep_states=False):
    """Bidirectional (Vision Mamba) scan forward; returns out (batch, dim, L).  With keep_states the
    given workspace keeps what vim_bidir_bwd(..., workspace_has_states=True) needs."""
    return VimForwardPlan(u, delta, A, B, C, D, delta_bias, z, delta_softplus, workspace,
                          keep_states=keep_states).run()


def vim_bidir_bwd(u, delta, A, B, C, D=None, delta_bias=None, z=None, dout=None, delta_softplus=True,
                  workspace=None, workspace_has_states=False):
    """Backward of vim_bidir_fwd; returns a dict of gradients (None for absent inputs).  With
    workspace_has_states, `workspace` must be the one a forward with keep_states=True used for the
    same inputs (the forward is then not recomputed)."""
    u, delta, dout = _c(u), _c(delta), _c(dout)
    dev = _dev(u)
    B, C, z = _c(B), _c(C), _c(z)
    A = _c(A, torch.float32)
    D = _c(D, torch.float32)
    delta_bias = _c(delta_bias, torch.float32)
    batch, K, dim, L = u.shape
    if K != 2:
        raise SS2DError("u must be (batch, 2, dim, L)")
    N = A.shape[-1]
    du, ddelta = torch.empty_like(u), torch.empty_like(delta)
    dA = torch.empty_like(A)
    dB, dC = torch.empty_like(B), torch.empty_like(C)
    dD = torch.empty_like(D) if D is not None else None
    dbias = torch.empty_like(delta_bias) if delta_bias is not None else None
    dz = torch.empty_like(z) if z is not None else None
    ws = _workspace(vim_bidir_workspace_bytes(batch, dim, L, N, u.dtype), dev, workspace)
    a = VimBwdArgs(u=_ptr(u), delta=_ptr(delta), A=_ptr(A), Bm=_ptr(B), Cm=_ptr(C), Dskip=_ptr(D),
                   delta_bias=_ptr(delta_bias), z=_ptr(z), dout=_ptr(dout), du=_ptr(du), ddelta=_ptr(ddelta),
                   dA=_ptr(dA), dBm=_ptr(dB), dCm=_ptr(dC), dDskip=_ptr(dD), ddelta_bias=_ptr(dbias), dz=_ptr(dz),
                   workspace=_ptr(ws), workspace_bytes=ws.numel() * ws.element_size(), batch=batch, dim=dim,
                   seqlen=L, dstate=N, dtype=_dtype_code(u.dtype), delta_softplus=int(bool(delta_softplus)),
                   workspace_has_states=int(bool(workspace_has_states)))
    if workspace_has_states and workspace is None:
        raise SS2DError("workspace_has_states needs the forward's workspace")
    _check(lib().vim_bidir_bwd(ctypes.byref(a), _stream(dev)), "vim_bidir_bwd")
    return {"du": du, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "ddelta_bias": dbias, "dz": dz}


def selective_scan_step(state, x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False):
    """One recurrent step from a carried state: `state` (batch, dim, N), a contiguous fp32 device
    tensor, is updated in place; x, delta, z are (batch, dim); B, C are (batch, G, N) or
    (batch, N).  Returns out (batch, dim)."""
    if state.dtype != torch.float32 or not state.is_contiguous():
        raise SS2DError("state must be a contiguous fp32 tensor (it is updated in place)")
    x, delta = _c(x), _c(delta)
    dev = _dev(x)
    if B.dim() == 2:
        B, C = B.unsqueeze(1), C.unsqueeze(1)
    B, C, z = _c(B), _c(C), _c(z)
    A = _c(A, torch.float32)
    D = _c(D, torch.float32)
    delta_bias = _c(delta_bias, torch.float32)
    batch, dim = x.shape
    N = A.shape[1]
    out = torch.empty_like(x)
    a = SsStepArgs(state=_ptr(state), x=_ptr(x), delta=_ptr(delta), A=_ptr(A), Bm=_ptr(B), Cm=_ptr(C), Dskip=_ptr(D),
                   z=_ptr(z), delta_bias=_ptr(delta_bias), out=_ptr(out), batch=batch, dim=dim, dstate=N,
                   ngroups=B.shape[1], dtype=_dtype_code(x.dtype), delta_softplus=int(bool(delta_softplus)))
    _check(lib().selective_scan_step(ctypes.byref(a), _stream(dev)), "selective_scan_step")
    return out
