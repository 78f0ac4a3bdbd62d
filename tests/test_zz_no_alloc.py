"""The allocation-free forward (ss2d_fwd_noalloc, for callers that cannot allocate): called
through the C ABI, it gives ss2d_fwd's result bit for bit (the same kernels, with the library's
fixed per-GPU scratch in place of the caller's workspace) on consecutive calls whose scratch
contents the previous call left behind (the second smaller than the first), and refuses problems
larger than its scratch with SS2D_ERR_TOO_LARGE without touching the output."""
import ctypes

import numpy as np
import pytest
import torch

import selective_scan_amd as ss
from gpu_util import to_dev
from selective_scan_amd import _binding as bnd
from selective_scan_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(batch, H, W, dim, N, dtype, seed, k=0, ln=False, R=0):
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, dtype, has_z=True, seed_base=seed)
    t = dict(x=to_dev(inp["x"], dtype), A=to_dev(inp["A"], "f32"), D=to_dev(inp["D"], "f32"),
             delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dtype))
    if R:
        pw = synth.make_proj_params(dim, N, R, seed_base=seed)
        t.update(delta=None, B=None, C=None, x_proj_w=to_dev(pw["x_proj_w"], "f32"),
                 dt_proj_w=to_dev(pw["dt_proj_w"], "f32"))
    else:
        t.update(delta=to_dev(inp["delta"], dtype), B=to_dev(inp["B"], dtype), C=to_dev(inp["C"], dtype))
    if k:
        fp = synth.make_front_params(dim, k, seed_base=seed)
        t.update(conv_w=to_dev(fp["conv_w"], "f32"), conv_b=to_dev(fp["conv_b"], "f32"))
    if ln:
        lp = synth.make_ln_params(dim, seed_base=seed)
        t.update(layer_norm=True, ln_w=to_dev(lp["ln_w"], "f32"), ln_b=to_dev(lp["ln_b"], "f32"))
    return t


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc_abi(t, out):
    """ss2d_fwd_noalloc through the C ABI; returns its status."""
    x = t["x"]
    batch, dim, H, W = x.shape
    R = t["dt_proj_w"].shape[-1] if t.get("dt_proj_w") is not None else 0
    conv_w = t.get("conv_w")
    a = bnd.SS2DFwdArgs(x=_p(x), delta=_p(t["delta"]), A=_p(t["A"]), Bm=_p(t["B"]), Cm=_p(t["C"]), Dskip=_p(t["D"]),
                        delta_bias=_p(t["delta_bias"]), z=_p(t["z"]), out=_p(out), workspace=None, workspace_bytes=0,
                        batch=batch, dim=dim, height=H, width=W, dstate=t["A"].shape[-1],
                        dtype=bnd.DTYPE_F32 if x.dtype == torch.float32 else bnd.DTYPE_BF16, delta_softplus=1,
                        keep_states=0, conv_w=_p(conv_w), conv_b=_p(t.get("conv_b")),
                        conv_k=0 if conv_w is None else conv_w.shape[-1], layer_norm=int(t.get("layer_norm", False)),
                        ln_w=_p(t.get("ln_w")), ln_b=_p(t.get("ln_b")), ln_eps=1e-5, x_proj_w=_p(t.get("x_proj_w")),
                        dt_proj_w=_p(t.get("dt_proj_w")), dt_rank=R)
    return bnd.lib().ss2d_fwd_noalloc(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# Each case: two calls in a row on one GPU's scratch, the second smaller than the first.
CASES = {
    "stage1_b2_then_small": [(2, 56, 56, 192, 16, "bf16", 0, False, 0), (1, 28, 28, 96, 16, "bf16", 0, False, 0)],
    "chunked_then_ragged": [(1, 64, 64, 64, 16, "f32", 0, False, 0), (2, 9, 11, 24, 16, "bf16", 0, False, 0)],
    "front_ln_then_producer": [(2, 14, 14, 96, 16, "bf16", 3, True, 0), (2, 13, 15, 16, 16, "f32", 3, True, 3)],
    "stage3_b8_then_b3": [(8, 14, 14, 768, 16, "bf16", 0, False, 0), (3, 14, 14, 768, 16, "bf16", 0, False, 0)],
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_ss2d_fwd_on_consecutive_calls(name):
    for i, (batch, H, W, dim, N, dtype, k, ln, R) in enumerate(CASES[name]):
        print(f"ss2d_fwd_noalloc {name} call {i}: {batch}x{dim}x{H}x{W} N={N} {dtype} k={k} ln={ln} R={R}", flush=True)
        t = _inputs(batch, H, W, dim, N, dtype, seed=3000 + 17 * i + H, k=k, ln=ln, R=R)
        need = ss.ss2d_workspace_bytes(batch, dim, H, W, N, t["x"].dtype, R)
        assert need <= ss.ss2d_fwd_noalloc_max_workspace_bytes()
        out = torch.empty_like(t["x"])
        assert _noalloc_abi(t, out) == bnd.SS2D_OK
        ref = ss.ss2d_fwd(**t)  # the existing entry point with its own workspace
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (name, i)


def test_noalloc_repeat_after_other_shape_and_plane_path():
    """A call, a call of another shape, the first again: the same result (nothing relies on what
    the scratch holds); a one-kernel-per-plane call (state size 4) larger than the scratch runs,
    since it needs none."""
    t1 = _inputs(2, 20, 24, 40, 16, "bf16", seed=3100)
    t2 = _inputs(1, 31, 17, 12, 8, "f32", seed=3101)
    o1, o2, o3 = torch.empty_like(t1["x"]), torch.empty_like(t2["x"]), torch.empty_like(t1["x"])
    assert _noalloc_abi(t1, o1) == 0 and _noalloc_abi(t2, o2) == 0 and _noalloc_abi(t1, o3) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)
    assert torch.equal(o2, ss.ss2d_fwd(**t2))
    big = _inputs(64, 56, 56, 48, 4, "bf16", seed=3102)
    assert ss.ss2d_workspace_bytes(64, 48, 56, 56, 4, torch.bfloat16) > ss.ss2d_fwd_noalloc_max_workspace_bytes()
    ob = torch.empty_like(big["x"])
    assert _noalloc_abi(big, ob) == 0
    assert torch.equal(ob, ss.ss2d_fwd(**big))


def test_noalloc_rejects_too_large_without_launching():
    t = _inputs(4, 56, 56, 192, 16, "bf16", seed=3200)
    out = torch.full_like(t["x"], 7.0)
    assert _noalloc_abi(t, out) == bnd.SS2D_ERR_TOO_LARGE
    with pytest.raises(ss.SS2DError, match="too large"):
        ss.ss2d_fwd_noalloc(**t, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    np.testing.assert_equal(bnd.lib().ss2d_fwd_noalloc_max_workspace_bytes(), 128 << 20)
