"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/ss2d.h declares, the binding's argument blocks match the header's struct layouts, and
invalid arguments are rejected with the documented status before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ss2d.h")


@pytest.fixture(scope="module")
def lib():
    from selective_scan_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from selective_scan_amd import build
        build.build()
    return _binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"ss2d_cross_scan", "ss2d_cross_merge", "selective_scan_fwd", "selective_scan_bwd", "ss2d_fwd",
            "ss2d_bwd", "ss2d_fwd_stage", "selective_scan_workspace_bytes", "ss2d_workspace_bytes",
            "ss2d_abi_version", "ss2d_status_string", "vim_bidir_workspace_bytes", "vim_bidir_fwd",
            "ss2d_proj_workspace_bytes",
            "vim_bidir_fwd_stage", "vim_bidir_bwd", "selective_scan_step", "ss2d_fwd_single_kernel",
            "ss2d_fwd_noalloc", "ss2d_fwd_noalloc_max_workspace_bytes"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(lib, n)


def test_version_and_status_strings(lib):
    assert lib.ss2d_abi_version() == 8
    assert lib.ss2d_status_string(0) == b"ok"
    assert b"too large" in lib.ss2d_status_string(4)
    assert b"invalid" in lib.ss2d_status_string(1)
    assert b"unsupported" in lib.ss2d_status_string(2)
    assert lib.ss2d_status_string(99) == b"unknown status"


STRUCTS = {"ss_fwd_args": "SsFwdArgs", "ss_bwd_args": "SsBwdArgs", "ss2d_fwd_args": "SS2DFwdArgs",
           "ss2d_bwd_args": "SS2DBwdArgs", "vim_bidir_fwd_args": "VimFwdArgs", "vim_bidir_bwd_args": "VimBwdArgs",
           "ss_step_args": "SsStepArgs"}


def test_binding_structs_match_header(tmp_path):
    """Compile a probe against the header with the host C compiler and compare every field offset."""
    from selective_scan_amd import _binding
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ss2d.h"', "int main(void) {"]
    for cname, pyname in STRUCTS.items():
        st = getattr(_binding, pyname)
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in st._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.check_call(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
                           "/opt/rocm/include", str(src), "-o", str(exe)])
    out = subprocess.check_output([str(exe)], text=True).split("\n")
    got = {}
    for line in out:
        if line:
            s, f, v = line.split()
            got[(s, f)] = int(v)
    for cname, pyname in STRUCTS.items():
        st = getattr(_binding, pyname)
        assert got[(cname, "size")] == ctypes.sizeof(st), cname
        for f, _ in st._fields_:
            assert got[(cname, f)] == getattr(st, f).offset, (cname, f)


def _fwd_args(**kw):
    from selective_scan_amd._binding import SsFwdArgs
    base = dict(u=0x1000, delta=0x2000, A=0x3000, Bm=0x4000, Cm=0x5000, out=0x6000, batch=2, dim=8, dstate=4,
                seqlen=16, ngroups=1, dtype=0, delta_softplus=1)
    base.update(kw)
    return SsFwdArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(dstate=0), 2), (dict(dstate=65), 2), (dict(dtype=7), 2), (dict(ngroups=3), 1), (dict(ngroups=0), 1),
    (dict(batch=-1), 1), (dict(u=0), 1), (dict(out=0), 1), (dict(A=0), 1), (dict(u=0x1001), 1),
    (dict(workspace=0x10000, workspace_bytes=16), 1),
])
def test_selective_scan_fwd_rejects(lib, kw, status):
    a = _fwd_args(**kw)
    assert lib.selective_scan_fwd(ctypes.byref(a), None) == status


def test_selective_scan_fwd_empty_is_noop(lib):
    assert lib.selective_scan_fwd(ctypes.byref(_fwd_args(batch=0, u=0, delta=0, out=0)), None) == 0
    assert lib.selective_scan_fwd(ctypes.byref(_fwd_args(seqlen=0)), None) == 0
    assert lib.selective_scan_fwd(None, None) == 1


def test_selective_scan_bwd_rejects(lib):
    from selective_scan_amd._binding import SsBwdArgs
    base = dict(u=0x1000, delta=0x2000, A=0x3000, Bm=0x4000, Cm=0x5000, dout=0x6000, du=0x7000, ddelta=0x8000,
                dA=0x9000, dBm=0xa000, dCm=0xb000, workspace=0x10000, workspace_bytes=1, batch=2, dim=8,
                dstate=4, seqlen=16, ngroups=1, dtype=0, delta_softplus=1)
    assert lib.selective_scan_bwd(ctypes.byref(SsBwdArgs(**base)), None) == 1           # workspace too small
    assert lib.selective_scan_bwd(ctypes.byref(SsBwdArgs(**{**base, "z": 0xc000})), None) == 1  # z without dz
    assert lib.selective_scan_bwd(ctypes.byref(SsBwdArgs(**{**base, "dstate": 100})), None) == 2
    assert lib.selective_scan_bwd(ctypes.byref(SsBwdArgs(**{**base, "dim": 0})), None) == 0


def test_ss2d_rejects(lib):
    from selective_scan_amd._binding import SS2DBwdArgs, SS2DFwdArgs
    f = dict(x=0x1000, delta=0x2000, A=0x3000, Bm=0x4000, Cm=0x5000, out=0x6000, workspace=0x10000,
             workspace_bytes=1, batch=1, dim=4, height=3, width=5, dstate=4, dtype=1, delta_softplus=1)
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**f)), None) == 1                       # workspace too small
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**f, "workspace": 0})), None) == 1
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**f, "dtype": 3})), None) == 2
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**f, "height": 0})), None) == 0       # empty map
    assert lib.ss2d_fwd_stage(ctypes.byref(SS2DFwdArgs(**f)), 3, None) == 1               # bad stage
    b = dict(x=0x1000, delta=0x2000, A=0x3000, Bm=0x4000, Cm=0x5000, dout=0x6000, dx=0x7000, ddelta=0x8000,
             dA=0x9000, dBm=0xa000, dCm=0xb000, workspace=0x10000, workspace_bytes=1, batch=1, dim=4, height=3,
             width=5, dstate=4, dtype=0, delta_softplus=1)
    assert lib.ss2d_bwd(ctypes.byref(SS2DBwdArgs(**b)), None) == 1
    assert lib.ss2d_bwd(ctypes.byref(SS2DBwdArgs(**{**b, "Dskip": 0xc000})), None) == 1  # D without dD
    # the input front: odd filter sizes 1..7 only, a bias needs a filter, gradients need outputs
    for k, st in ((2, 2), (9, 2), (0, 2), (-3, 2)):
        assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**f, "conv_w": 0xd000, "conv_k": k})), None) == st, k
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**f, "conv_b": 0xe000, "conv_k": 3})), None) == 1
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**f, "conv_w": 0xd002, "conv_k": 3})), None) == 1
    big = dict(workspace_bytes=1 << 40, dz=0, conv_w=0xd000, conv_k=3)
    assert lib.ss2d_bwd(ctypes.byref(SS2DBwdArgs(**{**b, **big})), None) == 1                 # no dconv_w
    assert lib.ss2d_bwd(ctypes.byref(SS2DBwdArgs(**{**b, **big, "dconv_w": 0xf000, "conv_b": 0xe000})),
                        None) == 1                                                            # no dconv_b
    # the LayerNorm: eps finite and >= 0, aligned parameters, gradients need outputs
    for eps in (-1.0, float("nan"), float("inf")):
        assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**f, "layer_norm": 1, "ln_eps": eps})), None) == 1, eps
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**f, "layer_norm": 1, "ln_w": 0xd001})), None) == 1
    ln = dict(workspace_bytes=1 << 40, dz=0, layer_norm=1, ln_eps=1e-5)
    assert lib.ss2d_bwd(ctypes.byref(SS2DBwdArgs(**{**b, **ln, "ln_w": 0xd000})), None) == 1        # no dln_w
    assert lib.ss2d_bwd(ctypes.byref(SS2DBwdArgs(**{**b, **ln, "ln_b": 0xd000})), None) == 1        # no dln_b
    # the Δ/B/C producer: both weights, dt_rank in [1, dim], weight gradients required
    pf = {**f, "delta": 0, "Bm": 0, "Cm": 0, "workspace_bytes": 1 << 40}
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**pf, "x_proj_w": 0xd000, "dt_rank": 2})), None) == 1  # no dt_proj_w
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**pf, "dt_proj_w": 0xd000, "dt_rank": 2})), None) == 1  # no x_proj_w
    for r in (0, 5):
        assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**pf, "x_proj_w": 0xd000, "dt_proj_w": 0xe000, "dt_rank": r})),
                            None) == 1, r
    assert lib.ss2d_fwd(ctypes.byref(SS2DFwdArgs(**{**f, "delta": 0})), None) == 1    # no delta, no producer
    pb = {**b, "delta": 0, "Bm": 0, "Cm": 0, "ddelta": 0, "dBm": 0, "dCm": 0, "workspace_bytes": 1 << 40,
          "x_proj_w": 0xd000, "dt_proj_w": 0xe000, "dt_rank": 2}
    assert lib.ss2d_bwd(ctypes.byref(SS2DBwdArgs(**pb)), None) == 1                   # no weight gradients


def test_ss2d_single_kernel_query(lib):
    """Which ss2d_fwd calls run as one kernel per plane (host logic only, nothing enqueued)."""
    from selective_scan_amd._binding import SS2DFwdArgs
    f = dict(x=0x1000, delta=0x2000, A=0x3000, Bm=0x4000, Cm=0x5000, out=0x6000, workspace=0x10000,
             workspace_bytes=1 << 40, batch=2, dim=4, height=8, width=8, dstate=1, dtype=1, delta_softplus=1)

    def q(**kw):
        return lib.ss2d_fwd_single_kernel(ctypes.byref(SS2DFwdArgs(**{**f, **kw})))

    for n, want in ((1, 1), (2, 1), (4, 1), (3, 0), (8, 0), (16, 0)):
        assert q(dstate=n) == want, n
    assert q(dtype=0, z=0x7000, Dskip=0x8000, delta_bias=0x9000, delta_softplus=0) == 1
    assert q(height=56, width=56) == 1
    assert q(height=63, width=64) == 1        # L = 4032: the largest plane within 63 KB
    assert q(height=3, width=5) == 0          # L not a multiple of 8
    assert q(height=64, width=64) == 0        # the plane's LDS arrays exceed 63 KB
    assert q(x=0x1008) == 0                   # an I/O tensor not 16-byte aligned
    assert q(z=0x7008) == 0
    assert q(keep_states=1) == 0
    assert q(layer_norm=1, ln_eps=1e-5) == 0
    assert q(conv_w=0xd000, conv_k=3) == 0
    assert q(delta=0, Bm=0, Cm=0, x_proj_w=0xd000, dt_proj_w=0xe000, dt_rank=2) == 0
    assert q(workspace_bytes=1) == 0          # invalid arguments
    assert q(height=0) == 0                   # empty map
    assert q(dtype=3) == 0


def test_vim_bidir_rejects(lib):
    from selective_scan_amd._binding import VimBwdArgs, VimFwdArgs
    f = dict(u=0x1000, delta=0x2000, A=0x3000, Bm=0x4000, Cm=0x5000, out=0x6000, workspace=0x10000,
             workspace_bytes=1, batch=1, dim=4, seqlen=7, dstate=4, dtype=1, delta_softplus=1)
    assert lib.vim_bidir_fwd(ctypes.byref(VimFwdArgs(**f)), None) == 1                    # workspace too small
    assert lib.vim_bidir_fwd(ctypes.byref(VimFwdArgs(**{**f, "workspace": 0})), None) == 1
    assert lib.vim_bidir_fwd(ctypes.byref(VimFwdArgs(**{**f, "dtype": 3})), None) == 2
    assert lib.vim_bidir_fwd(ctypes.byref(VimFwdArgs(**{**f, "dstate": 65})), None) == 2
    assert lib.vim_bidir_fwd(ctypes.byref(VimFwdArgs(**{**f, "seqlen": -1})), None) == 1
    assert lib.vim_bidir_fwd(ctypes.byref(VimFwdArgs(**{**f, "u": 0x1001})), None) == 1    # misaligned bf16
    assert lib.vim_bidir_fwd(ctypes.byref(VimFwdArgs(**{**f, "seqlen": 0})), None) == 0    # empty
    assert lib.vim_bidir_fwd(None, None) == 1
    assert lib.vim_bidir_fwd_stage(ctypes.byref(VimFwdArgs(**f)), 5, None) == 1           # bad stage
    assert lib.vim_bidir_fwd_stage(ctypes.byref(VimFwdArgs(**{**f, "seqlen": 0})), 0, None) == 0
    b = dict(u=0x1000, delta=0x2000, A=0x3000, Bm=0x4000, Cm=0x5000, dout=0x6000, du=0x7000, ddelta=0x8000,
             dA=0x9000, dBm=0xa000, dCm=0xb000, workspace=0x10000, workspace_bytes=1, batch=1, dim=4, seqlen=7,
             dstate=4, dtype=0, delta_softplus=1)
    assert lib.vim_bidir_bwd(ctypes.byref(VimBwdArgs(**b)), None) == 1                    # workspace too small
    assert lib.vim_bidir_bwd(ctypes.byref(VimBwdArgs(**{**b, "z": 0xc000})), None) == 1   # z without dz
    assert lib.vim_bidir_bwd(ctypes.byref(VimBwdArgs(**{**b, "dim": 0})), None) == 0


def test_selective_scan_step_rejects(lib):
    from selective_scan_amd._binding import SsStepArgs
    a = dict(state=0x1000, x=0x2000, delta=0x3000, A=0x4000, Bm=0x5000, Cm=0x6000, out=0x7000, batch=2, dim=8,
             dstate=16, ngroups=2, dtype=1, delta_softplus=1)
    assert lib.selective_scan_step(ctypes.byref(SsStepArgs(**{**a, "state": 0})), None) == 1
    assert lib.selective_scan_step(ctypes.byref(SsStepArgs(**{**a, "ngroups": 3})), None) == 1
    assert lib.selective_scan_step(ctypes.byref(SsStepArgs(**{**a, "dstate": 0})), None) == 2
    assert lib.selective_scan_step(ctypes.byref(SsStepArgs(**{**a, "dtype": 2})), None) == 2
    assert lib.selective_scan_step(ctypes.byref(SsStepArgs(**{**a, "x": 0x2001})), None) == 1   # misaligned bf16
    assert lib.selective_scan_step(ctypes.byref(SsStepArgs(**{**a, "state": 0x1002})), None) == 1
    assert lib.selective_scan_step(ctypes.byref(SsStepArgs(**{**a, "batch": 0})), None) == 0    # empty
    assert lib.selective_scan_step(None, None) == 1


def test_cross_scan_merge_reject(lib):
    assert lib.ss2d_cross_scan(None, None, 1, 1, 2, 2, 0, None) == 1
    assert lib.ss2d_cross_scan(0x1000, 0x2000, 1, 1, 2, 2, 5, None) == 2
    assert lib.ss2d_cross_scan(0x1000, 0x2000, -1, 1, 2, 2, 0, None) == 1
    assert lib.ss2d_cross_scan(None, None, 0, 1, 2, 2, 0, None) == 0   # empty: nothing to do
    assert lib.ss2d_cross_merge(0x1001, 0x2000, 1, 1, 2, 2, 0, None) == 1  # misaligned fp32


def test_workspace_queries(lib):
    a = lib.selective_scan_workspace_bytes(2, 64, 16, 256, 1)
    b = lib.selective_scan_workspace_bytes(2, 64, 16, 512, 1)
    assert 0 < a < b
    assert lib.selective_scan_workspace_bytes(2, 64, 0, 256, 1) == 0
    s1 = lib.ss2d_workspace_bytes(1, 16, 8, 8, 4, 0)
    s2 = lib.ss2d_workspace_bytes(1, 16, 8, 8, 4, 1)
    assert 0 < s2 <= s1  # fp32 intermediates: the I/O type changes no workspace region
    assert lib.ss2d_workspace_bytes(1, 16, 8, 8, 4, 9) == 0
    p1 = lib.ss2d_proj_workspace_bytes(1, 16, 8, 8, 4, 2, 1)
    assert p1 > s2 and p1 % 256 == 0  # the plain regions plus the producer's
    assert lib.ss2d_proj_workspace_bytes(1, 16, 8, 8, 4, 0, 1) == 0
    assert lib.ss2d_proj_workspace_bytes(1, 16, 8, 8, 4, 17, 1) == 0
    v1 = lib.vim_bidir_workspace_bytes(2, 8, 197, 16, 1)
    v2 = lib.vim_bidir_workspace_bytes(2, 8, 197, 16, 0)
    assert 0 < v1 == v2  # fp32 direction outputs and gradients: the same size for either I/O type
    assert lib.vim_bidir_workspace_bytes(2, 8, 197, 0, 1) == 0
    assert lib.vim_bidir_workspace_bytes(2, 8, 197, 16, 4) == 0
    assert all(v % 256 == 0 for v in (a, b, s1, s2, v1, v2))


def test_ss2d_fwd_noalloc_host_checks(lib):
    """The allocation-free forward: its scratch size, and what it rejects before touching the GPU
    (invalid arguments, kept states, problems larger than the scratch)."""
    from selective_scan_amd._binding import SS2DFwdArgs
    cap = lib.ss2d_fwd_noalloc_max_workspace_bytes()
    assert cap == 128 << 20
    f = dict(x=0x1000, delta=0x2000, A=0x3000, Bm=0x4000, Cm=0x5000, out=0x6000, batch=4, dim=192, height=56,
             width=56, dstate=16, dtype=1, delta_softplus=1)
    assert lib.ss2d_workspace_bytes(4, 192, 56, 56, 16, 1) > cap
    assert lib.ss2d_fwd_noalloc(ctypes.byref(SS2DFwdArgs(**f)), None) == 4              # too large
    assert lib.ss2d_fwd_noalloc(ctypes.byref(SS2DFwdArgs(**{**f, "keep_states": 1})), None) == 1
    assert lib.ss2d_fwd_noalloc(ctypes.byref(SS2DFwdArgs(**{**f, "x": 0})), None) == 1
    assert lib.ss2d_fwd_noalloc(ctypes.byref(SS2DFwdArgs(**{**f, "dtype": 5})), None) == 2
    assert lib.ss2d_fwd_noalloc(ctypes.byref(SS2DFwdArgs(**{**f, "batch": 0})), None) == 0  # empty
    assert lib.ss2d_fwd_noalloc(None, None) == 1


# Every exported prototype of include/ss2d.h: name -> parameter types (names dropped, whitespace
# normalised).  A change to the boundary must change this table too.
SIGNATURES = {
    "ss2d_abi_version": ("int", ("void",)),
    "ss2d_status_string": ("const char*", ("int",)),
    "ss2d_cross_scan": ("int", ("const void*", "void*", "int64_t", "int64_t", "int64_t", "int64_t", "int",
                                "hipStream_t")),
    "ss2d_cross_merge": ("int", ("const void*", "void*", "int64_t", "int64_t", "int64_t", "int64_t", "int",
                                 "hipStream_t")),
    "selective_scan_workspace_bytes": ("size_t", ("int64_t",) * 5),
    "selective_scan_fwd": ("int", ("const ss_fwd_args*", "hipStream_t")),
    "selective_scan_bwd": ("int", ("const ss_bwd_args*", "hipStream_t")),
    "selective_scan_step": ("int", ("const ss_step_args*", "hipStream_t")),
    "ss2d_proj_workspace_bytes": ("size_t", ("int64_t",) * 6 + ("int",)),
    "ss2d_workspace_bytes": ("size_t", ("int64_t",) * 5 + ("int",)),
    "ss2d_fwd": ("int", ("const ss2d_fwd_args*", "hipStream_t")),
    "ss2d_fwd_single_kernel": ("int", ("const ss2d_fwd_args*",)),
    "ss2d_fwd_noalloc_max_workspace_bytes": ("size_t", ("void",)),
    "ss2d_fwd_noalloc": ("int", ("const ss2d_fwd_args*", "hipStream_t")),
    "ss2d_fwd_stage": ("int", ("const ss2d_fwd_args*", "int", "hipStream_t")),
    "ss2d_bwd": ("int", ("const ss2d_bwd_args*", "hipStream_t")),
    "vim_bidir_workspace_bytes": ("size_t", ("int64_t",) * 4 + ("int",)),
    "vim_bidir_fwd": ("int", ("const vim_bidir_fwd_args*", "hipStream_t")),
    "vim_bidir_fwd_stage": ("int", ("const vim_bidir_fwd_args*", "int", "hipStream_t")),
    "vim_bidir_bwd": ("int", ("const vim_bidir_bwd_args*", "hipStream_t")),
}


def _prototypes():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*((?:const\s+)?\w+\s*\**)\s*(\w+)\s*\(([^)]*)\)\s*;", text, flags=re.M):
        ret, name, params = re.sub(r"\s+", "", m.group(1)), m.group(2), m.group(3)
        types = []
        for prm in params.split(","):
            prm = " ".join(prm.split())
            if prm == "void":
                types.append("void")
                continue
            # drop the parameter name: the last identifier
            t = re.sub(r"\s*\b\w+$", "", prm).replace(" *", "*")
            types.append(t)
        out[name] = (ret.replace("constchar", "const char"), tuple(types))
    return out


def test_exported_signatures():
    got = _prototypes()
    assert set(got) == set(SIGNATURES), sorted(set(got) ^ set(SIGNATURES))
    for name, want in SIGNATURES.items():
        assert got[name] == want, (name, got[name])
