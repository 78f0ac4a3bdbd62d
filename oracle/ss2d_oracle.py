"""fp64 CPU oracle of the SS2D path (TEST INFRASTRUCTURE ONLY; see oracle/__init__.py).

Sources (the pages the method is defined on):
  * SS2D as three steps -- cross-scan along four traversal routes, one S6 scan per
    route, cross-merge back to the 2-D map: VMamba paper translation (blog.csdn.net),
    section "2-D selective scan (SS2D) for visual data" and the caption of Fig. 2;
    the merge adds the four directional results: freeymw.com page, section 1.
  * The four routes are taken as row-major, column-major and both reversed, each a
    single sequence of length L = H*W (the plainest reading; the pages name the
    routes but print no index formula).
  * The selective scan itself: `selective_scan_ref` on the freeymw.com page, section 2
    (the C part of this oracle, ss_oracle.c).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ss_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libss_oracle.so")
_lib = None


def build_oracle_lib(force: bool = False) -> str:
    """Compile ss_oracle.c with gcc (IEEE double, OpenMP over independent rows)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _get_lib():
    global _lib
    if _lib is None:
        path = build_oracle_lib()
        lib = ctypes.CDLL(path)
        dp = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_ss_fwd.argtypes = [dp] * 8 + [ctypes.c_int] + [i64] * 5 + [dp] * 3
        lib.oracle_ss_fwd.restype = None
        lib.oracle_ss_bwd.argtypes = [dp] * 8 + [ctypes.c_int] + [i64] * 5 + [dp] * 9
        lib.oracle_ss_bwd.restype = None
        _lib = lib
    return _lib


def set_num_threads(n: int) -> int:
    """Threads of the C part's OpenMP loops from now on (for timing); returns the previous count.
    Threading only: each row is computed by one thread in the same order whatever the count."""
    lib = _get_lib()
    lib.omp_get_max_threads.restype = ctypes.c_int
    prev = int(lib.omp_get_max_threads())
    lib.omp_set_num_threads(ctypes.c_int(int(n)))
    return prev


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def softplus(x):
    """log(1 + e^x), exact form (F.softplus with its default settings)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


# ----------------------------------------------------------------------------------
# Selective scan (S6), generic shapes of `selective_scan_ref`
# ----------------------------------------------------------------------------------
def ss_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
           return_last_state=False, return_ypre=False):
    """Selective scan forward in fp64.

    u, delta, z: (batch, dim, L); A: (dim, N); B, C: (batch, G, N, L) or (batch, N, L)
    (read as G = 1); D, delta_bias: (dim,).  Returns out (batch, dim, L) and, on
    request, last_state (batch, dim, N) and the pre-gate output y + D*u.
    """
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias = map(_f64, (D, z, delta_bias))
    if B.ndim == 3:
        B = B[:, None]
    if C.ndim == 3:
        C = C[:, None]
    B = np.ascontiguousarray(B)
    C = np.ascontiguousarray(C)
    batch, dim, L = u.shape
    N = A.shape[1]
    G = B.shape[1]
    assert dim % G == 0 and A.shape == (dim, N) and B.shape == (batch, G, N, L) and C.shape == B.shape
    out = np.empty((batch, dim, L))
    last = np.empty((batch, dim, N)) if return_last_state else None
    ypre = np.empty((batch, dim, L)) if return_ypre else None
    _get_lib().oracle_ss_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                             _ptr(delta_bias), int(bool(delta_softplus)), batch, dim, N, L, G,
                             _ptr(out), _ptr(last), _ptr(ypre))
    res = [out]
    if return_last_state:
        res.append(last)
    if return_ypre:
        res.append(ypre)
    return res[0] if len(res) == 1 else tuple(res)


def ss_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, dout=None):
    """Exact gradient of ss_fwd w.r.t. every input, given dL/dout.

    Returns a dict with du, ddelta (w.r.t. the raw delta), dA, dB, dC and, when the
    corresponding input is given, dD, dz, ddelta_bias.
    """
    u, delta, A, B, C, dout = map(_f64, (u, delta, A, B, C, dout))
    D, z, delta_bias = map(_f64, (D, z, delta_bias))
    squeeze = B.ndim == 3
    if B.ndim == 3:
        B = np.ascontiguousarray(B[:, None])
        C = np.ascontiguousarray(C[:, None])
    batch, dim, L = u.shape
    N = A.shape[1]
    G = B.shape[1]
    du = np.empty_like(u)
    ddelta = np.empty_like(u)
    dA = np.empty((dim, N))
    dB = np.empty_like(B)
    dC = np.empty_like(C)
    dD = np.empty(dim) if D is not None else None
    dz = np.empty_like(u) if z is not None else None
    dbias = np.empty(dim) if delta_bias is not None else None
    _get_lib().oracle_ss_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                             _ptr(delta_bias), int(bool(delta_softplus)), batch, dim, N, L, G,
                             _ptr(dout), _ptr(du), _ptr(ddelta), _ptr(dA), _ptr(dB), _ptr(dC),
                             _ptr(dD), _ptr(dz), _ptr(dbias))
    if squeeze:
        dB, dC = dB[:, 0], dC[:, 0]
    return {"du": du, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "dz": dz,
            "ddelta_bias": dbias}


# ----------------------------------------------------------------------------------
# Cross-scan / cross-merge (exact index permutations)
# ----------------------------------------------------------------------------------
def perm_indices(H: int, W: int) -> np.ndarray:
    """idx[k, t] = flat pixel h*W + w that direction k visits at step t.

    k=0 row-major, k=1 column-major (t = w*H + h), k=2 and k=3 the same two
    traversals run from the last pixel back to the first.
    """
    L = H * W
    t = np.arange(L, dtype=np.int64)
    row = t
    col = (t % H) * W + (t // H)
    return np.stack([row, col, row[::-1], col[::-1]])


def cross_scan(x):
    """x (B, C, H, W) -> xs (B, 4, C, H*W) with xs[:, k, :, t] = x at pixel idx[k, t]."""
    x = np.asarray(x)
    Bsz, Cch, H, W = x.shape
    flat = x.reshape(Bsz, Cch, H * W)
    idx = perm_indices(H, W)
    return np.stack([flat[:, :, idx[k]] for k in range(4)], axis=1)


def cross_merge(ys, H: int, W: int):
    """ys (B, 4, C, H*W) -> y (B, C, H, W): y at pixel p = sum_k ys[:, k, :, t] with idx[k, t] = p.

    Summed in fp64 in the order k = 0, 1, 2, 3.
    """
    ys = np.asarray(ys, dtype=np.float64)
    Bsz, K, Cch, L = ys.shape
    assert K == 4 and L == H * W
    idx = perm_indices(H, W)
    y = np.zeros((Bsz, Cch, L))
    for k in range(4):
        y[:, :, idx[k]] += ys[:, k]
    return y.reshape(Bsz, Cch, H, W)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def ss2d_fwd(x, delta, A, B, C, D=None, delta_bias=None, z=None, delta_softplus=True,
             return_merged=False):
    """SS2D forward: cross_scan(x) -> selective scan per route (group k for route k)
    -> cross_merge -> optional gate silu(z) on the merged map.

    x, z: (Bt, D, H, W); delta: (Bt, 4, D, L); A: (4, D, N); B, C: (Bt, 4, N, L);
    D, delta_bias: (4, D).  Returns out (Bt, D, H, W) in fp64 (and the merged,
    pre-gate map on request).
    """
    x = _f64(x)
    Bt, Dm, H, W = x.shape
    L = H * W
    N = np.asarray(A).shape[-1]
    xs = cross_scan(x).reshape(Bt, 4 * Dm, L)
    ys = ss_fwd(xs, np.reshape(delta, (Bt, 4 * Dm, L)), np.reshape(A, (4 * Dm, N)), B, C,
                D=None if D is None else np.reshape(D, (4 * Dm,)), z=None,
                delta_bias=None if delta_bias is None else np.reshape(delta_bias, (4 * Dm,)),
                delta_softplus=delta_softplus)
    merged = cross_merge(ys.reshape(Bt, 4, Dm, L), H, W)
    out = merged * _silu(_f64(z)) if z is not None else merged
    return (out, merged) if return_merged else out


def ss2d_bwd(x, delta, A, B, C, D=None, delta_bias=None, z=None, dout=None, delta_softplus=True):
    """Exact gradient of ss2d_fwd (chain rule through the permutations).

    merge is the transpose of scan, so the gradient reaching route k is
    cross_scan(dL/dmerged) and dL/dx = cross_merge(du).  The gate's gradient is
    dz = dout * merged * silu'(z).  Returns dx, ddelta (Bt,4,D,L), dA (4,D,N),
    dB, dC (Bt,4,N,L), dD, ddelta_bias (4,D), dz (Bt,D,H,W).
    """
    x = _f64(x)
    Bt, Dm, H, W = x.shape
    L = H * W
    N = np.asarray(A).shape[-1]
    dout = _f64(dout)
    if z is not None:
        _, merged = ss2d_fwd(x, delta, A, B, C, D, delta_bias, None, delta_softplus, return_merged=True)
        zz = _f64(z)
        s = 1.0 / (1.0 + np.exp(-zz))
        dmerged = dout * zz * s
        dz = dout * merged * s * (1.0 + zz * (1.0 - s))
    else:
        dmerged, dz = dout, None
    dys = cross_scan(dmerged).reshape(Bt, 4 * Dm, L)
    xs = cross_scan(x).reshape(Bt, 4 * Dm, L)
    g = ss_bwd(xs, np.reshape(delta, (Bt, 4 * Dm, L)), np.reshape(A, (4 * Dm, N)), B, C,
               D=None if D is None else np.reshape(D, (4 * Dm,)), z=None,
               delta_bias=None if delta_bias is None else np.reshape(delta_bias, (4 * Dm,)),
               delta_softplus=delta_softplus, dout=dys)
    dx = cross_merge(g["du"].reshape(Bt, 4, Dm, L), H, W)
    return {
        "dx": dx,
        "ddelta": g["ddelta"].reshape(Bt, 4, Dm, L),
        "dA": g["dA"].reshape(4, Dm, N),
        "dB": g["dB"],
        "dC": g["dC"],
        "dD": None if D is None else g["dD"].reshape(4, Dm),
        "ddelta_bias": None if delta_bias is None else g["ddelta_bias"].reshape(4, Dm),
        "dz": dz,
    }
