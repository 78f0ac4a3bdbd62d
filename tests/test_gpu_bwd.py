"""GPU parity of the backward paths (selective_scan_bwd, ss2d_bwd) against the fp64 oracle's
exact gradients: within 1e-3 relative, except the gradients stored in bf16 in a bf16 run (du,
ddelta, dB, dC, dz, dx), whose one rounding to bf16 alone is up to 2^-9: 2e-2, as for bf16 outputs.
The fp32-stored gradients (dA, dD, ddelta_bias) are held to 1e-3 in every run."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ss
from gpu_util import TOL_GRAD, f64, grad_tol, rel_err, to_dev, to_f64
from selective_scan_amd import synth

pytestmark = pytest.mark.gpu

GRADS = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias")
_tol = grad_tol


def _case(batch, dim, N, L, G, dtype, has_z, has_D, has_bias, softplus, seed):
    inp = synth.make_ss_inputs(batch, dim, N, L, G, dtype, has_z=has_z, seed_base=seed, with_dout=True)
    if not softplus:
        inp["delta"] = (inp["delta"] & np.uint16(0x7FFF)) if dtype == "bf16" else np.abs(inp["delta"])
    A = inp["A"] * np.float32(0.5 + np.random.default_rng(seed).random((dim, 1)))
    Dv = inp["D"] * np.float32(0.7)
    dev = dict(u=to_dev(inp["u"], dtype), delta=to_dev(inp["delta"], dtype), A=to_dev(A, "f32"),
               B=to_dev(inp["B"], dtype), C=to_dev(inp["C"], dtype), D=to_dev(Dv, "f32") if has_D else None,
               z=to_dev(inp["z"], dtype) if has_z else None,
               delta_bias=to_dev(inp["delta_bias"], "f32") if has_bias and softplus else None)
    ref = dict(u=f64(inp["u"], dtype), delta=f64(inp["delta"], dtype), A=A.astype(np.float64),
               B=f64(inp["B"], dtype), C=f64(inp["C"], dtype), D=Dv.astype(np.float64) if has_D else None,
               z=f64(inp["z"], dtype) if has_z else None,
               delta_bias=inp["delta_bias"].astype(np.float64) if has_bias and softplus else None)
    return dev, ref, to_dev(inp["dout"], dtype), f64(inp["dout"], dtype)


BWD_CASES = [
    # batch, dim, N, L, G, dtype, z, D, bias, softplus
    (2, 64, 16, 256, 1, "f32", True, True, True, True),
    (2, 96, 16, 200, 2, "f32", False, True, True, True),     # partial wave, ragged tile
    (1, 70, 4, 129, 1, "f32", True, True, False, True),      # L % 4 != 0
    (3, 32, 1, 300, 4, "f32", False, False, True, True),
    (1, 16, 3, 77, 1, "f32", True, False, False, False),     # no softplus, N padded
    (2, 64, 32, 96, 2, "f32", True, True, True, True),
    (1, 64, 64, 40, 1, "f32", True, True, True, True),
    (1, 64, 8, 2048, 1, "f32", True, True, True, True),      # few rows: chunked
    (2, 128, 16, 256, 2, "bf16", True, True, True, True),
    (2, 8, 16, 1, 1, "f32", True, True, True, True),         # L = 1
]


@pytest.mark.parametrize("ci", range(len(BWD_CASES)), ids=[str(c[:6]) for c in BWD_CASES])
def test_selective_scan_bwd(ci):
    batch, dim, N, L, G, dtype, z, D, bias, sp = BWD_CASES[ci]
    dev, ref, dout, dout64 = _case(batch, dim, N, L, G, dtype, z, D, bias, sp, seed=300 + ci)
    g = ss.selective_scan_bwd(**dev, dout=dout, delta_softplus=sp)
    r = oracle.ss_bwd(**ref, delta_softplus=sp, dout=dout64)
    for k in GRADS:
        if r[k] is None:
            assert g[k] is None
            continue
        e = rel_err(to_f64(g[k]), r[k])
        assert e <= _tol(dtype, k), (k, e)


def test_selective_scan_bwd_reuses_forward_states():
    dev, ref, dout, dout64 = _case(2, 64, 16, 512, 1, "f32", True, True, True, True, seed=399)
    batch, dim, L = dev["u"].shape
    ws = torch.empty(ss.selective_scan_workspace_bytes(batch, dim, 16, L, 1), dtype=torch.uint8, device="cuda")
    ss.selective_scan_fwd(**dev, delta_softplus=True, workspace=ws)
    g = ss.selective_scan_bwd(**dev, dout=dout, delta_softplus=True, workspace=ws, workspace_has_states=True)
    r = oracle.ss_bwd(**ref, delta_softplus=True, dout=dout64)
    for k in GRADS:
        assert rel_err(to_f64(g[k]), r[k]) <= TOL_GRAD, k


def _ss2d(batch, H, W, dim, N, dtype, z, seed):
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, dtype, has_z=z, seed_base=seed, with_dout=True)
    dev = dict(x=to_dev(inp["x"], dtype), delta=to_dev(inp["delta"], dtype), A=to_dev(inp["A"], "f32"),
               B=to_dev(inp["B"], dtype), C=to_dev(inp["C"], dtype), D=to_dev(inp["D"], "f32"),
               delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dtype) if z else None)
    ref = dict(x=f64(inp["x"], dtype), delta=f64(inp["delta"], dtype), A=inp["A"].astype(np.float64),
               B=f64(inp["B"], dtype), C=f64(inp["C"], dtype), D=inp["D"].astype(np.float64),
               delta_bias=inp["delta_bias"].astype(np.float64), z=f64(inp["z"], dtype) if z else None)
    return dev, ref, to_dev(inp["dout"], dtype), f64(inp["dout"], dtype)


SS2D_GRADS = ("dx", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz")
SS2D_BWD_CASES = [
    (1, 8, 8, 16, 4, "f32", True),
    (2, 7, 9, 20, 16, "f32", True),
    (2, 14, 14, 70, 16, "f32", False),
    (1, 3, 40, 64, 8, "bf16", True),
    (1, 64, 64, 64, 16, "f32", True),   # few rows: chunked
    (1, 1, 1, 8, 4, "f32", True),
    (2, 12, 8, 13, 16, "bf16", True),   # route outputs in 4-step blocks (H, W multiples of 4)
    (1, 8, 12, 9, 16, "f32", False),    # the same without the gate
    (1, 8, 4, 10, 32, "f32", True),     # blocked du and dB / dC partials, 32 states (4-step sub-intervals)
    (1, 4, 8, 7, 64, "bf16", True),     # 64 states: 2-step sub-intervals, du stored element by element
    (2, 8, 8, 40, 8, "bf16", False),    # one lane per channel, 40 of 64 lanes active
    (1, 16, 8, 40, 16, "bf16", True),   # dΔ rows of whole lines (L = 128): two 64-step windows, a partial channel block
    (1, 64, 64, 40, 16, "bf16", True),  # the same, few rows: chunked, windows cut at the chunk ends
]


@pytest.mark.parametrize("case", SS2D_BWD_CASES, ids=[str(c) for c in SS2D_BWD_CASES])
def test_ss2d_bwd(case):
    batch, H, W, dim, N, dtype, z = case
    dev, ref, dout, dout64 = _ss2d(batch, H, W, dim, N, dtype, z, seed=50 + H * W)
    g = ss.ss2d_bwd(**dev, dout=dout)
    r = oracle.ss2d_bwd(**ref, dout=dout64)
    for k in SS2D_GRADS:
        if r[k] is None:
            assert g[k] is None
            continue
        e = rel_err(to_f64(g[k]), r[k])
        assert e <= _tol(dtype, k), (k, e)


@pytest.mark.parametrize("case", [(1, 8, 8, 16, 4, "f32", True), (2, 7, 9, 20, 16, "f32", True),
                                  (1, 3, 40, 64, 8, "bf16", True), (1, 64, 64, 64, 16, "f32", True),
                                  (2, 14, 14, 70, 16, "f32", False), (2, 12, 8, 13, 16, "bf16", True),
                                  (1, 8, 12, 9, 16, "f32", False), (1, 8, 4, 10, 32, "f32", True),
                                  (2, 8, 8, 40, 8, "bf16", False), (1, 16, 8, 40, 16, "bf16", True),
                                  (1, 64, 64, 40, 16, "bf16", True)], ids=str)
def test_ss2d_bwd_reuses_forward_states(case):
    """A training forward (keep_states) then the backward on its workspace: the oracle's gradients,
    and bit for bit what the backward that recomputes the forward gives."""
    batch, H, W, dim, N, dtype, z = case
    dev, ref, dout, dout64 = _ss2d(batch, H, W, dim, N, dtype, z, seed=70 + H * W)
    ws = torch.empty(ss.ss2d_workspace_bytes(batch, dim, H, W, N, dev["x"].dtype), dtype=torch.uint8, device="cuda")
    out = ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
    g = ss.ss2d_bwd(**dev, dout=dout, workspace=ws, workspace_has_states=True)
    g2 = ss.ss2d_bwd(**dev, dout=dout)
    plan = ss.SS2DForwardPlan(**dev)  # the three stages without kept states: the same result, bit for bit
    for stage in (0, 1, 2):
        plan.run_stage(stage)
    assert torch.equal(out, plan.out)
    r = oracle.ss2d_bwd(**ref, dout=dout64)
    for k in SS2D_GRADS:
        if r[k] is None:
            assert g[k] is None
            continue
        assert torch.equal(g[k], g2[k]), k
        e = rel_err(to_f64(g[k]), r[k])
        assert e <= _tol(dtype, k), (k, e)


@pytest.mark.parametrize("params", synth.PARAMS)
def test_ss2d_bwd_tiny_config(params):
    cfg = synth.TINY
    inp = synth.make_config_inputs(cfg, with_dout=True, params=params)
    dev, ref = _dev_ref(inp, cfg.dtype, cfg.has_z)
    g = ss.ss2d_bwd(**dev, dout=to_dev(inp["dout"], cfg.dtype))
    r = oracle.ss2d_bwd(**ref, dout=f64(inp["dout"], cfg.dtype))
    for k in SS2D_GRADS:
        assert rel_err(to_f64(g[k]), r[k]) <= TOL_GRAD, k


def _dev_ref(inp, dt, has_z=True):
    dev = dict(x=to_dev(inp["x"], dt), delta=to_dev(inp["delta"], dt), A=to_dev(inp["A"], "f32"),
               B=to_dev(inp["B"], dt), C=to_dev(inp["C"], dt), D=to_dev(inp["D"], "f32"),
               delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dt) if has_z else None)
    ref = dict(x=f64(inp["x"], dt), delta=f64(inp["delta"], dt), A=inp["A"].astype(np.float64),
               B=f64(inp["B"], dt), C=f64(inp["C"], dt), D=inp["D"].astype(np.float64),
               delta_bias=inp["delta_bias"].astype(np.float64), z=f64(inp["z"], dt) if has_z else None)
    return dev, ref


@pytest.mark.parametrize("cfg", [synth.HIGHRES, synth.STAGE3], ids=lambda c: c.name)
def test_ss2d_bwd_config_full(cfg):
    """The high-resolution (128x128, B=4, D=192, N=16, fp32) and stage-3 (14x14, B=128, D=768,
    N=16, bf16) workloads at full size, in the benchmark's training launch configuration (forward
    with keep_states, backward on its states), against the oracle's full fp64 gradients.  A and D
    are drawn per route, channel and state."""
    inp = synth.make_config_inputs(cfg, with_dout=True, params="general")
    dev, ref = _dev_ref(inp, cfg.dtype, cfg.has_z)
    print(f"full-config backward {cfg.name}", flush=True)
    ws = torch.empty(ss.ss2d_workspace_bytes(cfg.batch, cfg.dim, cfg.height, cfg.width, cfg.dstate, dev["x"].dtype),
                     dtype=torch.uint8, device="cuda")
    ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
    g = ss.ss2d_bwd(**dev, dout=to_dev(inp["dout"], cfg.dtype), workspace=ws, workspace_has_states=True)
    got = {k: to_f64(g[k]) for k in SS2D_GRADS}
    del g, ws, dev
    torch.cuda.empty_cache()
    r = oracle.ss2d_bwd(**ref, dout=f64(inp["dout"], cfg.dtype))
    for k in SS2D_GRADS:
        e = rel_err(got[k], r[k])
        assert e <= _tol(cfg.dtype, k), (k, e)


def test_ss2d_bwd_stage1_full_size_training_path():
    """Stage-1 (B=128, 56x56, D=192, N=16, bf16) at full size in the benchmark's training launch
    configuration (forward with keep_states, backward on its states), A and D drawn per route,
    channel and state.  Checked on what the oracle can compute from slices (rows are independent,
    and dB/dC of an image sum over its channels only): every gradient of 8 whole images (the
    first, the last and 6 drawn ones); dA, dD, ddelta_bias of 24 channels (the first, the last and
    22 drawn ones) summed over all 128 images."""
    cfg = synth.STAGE1
    inp = synth.make_config_inputs(cfg, with_dout=True, params="general")
    dt = cfg.dtype
    dev = dict(x=to_dev(inp["x"], dt), delta=to_dev(inp["delta"], dt), A=to_dev(inp["A"], "f32"),
               B=to_dev(inp["B"], dt), C=to_dev(inp["C"], dt), D=to_dev(inp["D"], "f32"),
               delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dt))
    ws = torch.empty(ss.ss2d_workspace_bytes(cfg.batch, cfg.dim, cfg.height, cfg.width, cfg.dstate, dev["x"].dtype),
                     dtype=torch.uint8, device="cuda")
    ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
    g = ss.ss2d_bwd(**dev, dout=to_dev(inp["dout"], dt), workspace=ws, workspace_has_states=True)
    torch.cuda.synchronize()
    f = lambda a: synth.storage_to_f64(a, dt)

    def ref(bs, ds):
        return oracle.ss2d_bwd(x=f(inp["x"][bs][:, ds]), delta=f(inp["delta"][bs][:, :, ds]),
                               A=inp["A"][:, ds].astype(np.float64), B=f(inp["B"][bs]), C=f(inp["C"][bs]),
                               D=inp["D"][:, ds].astype(np.float64), delta_bias=inp["delta_bias"][:, ds].astype(np.float64),
                               z=f(inp["z"][bs][:, ds]), dout=f(inp["dout"][bs][:, ds]))

    rng = np.random.default_rng(21)
    images = np.unique(np.concatenate([[0, cfg.batch - 1], rng.choice(np.arange(1, cfg.batch - 1), 6, replace=False)]))
    r = ref(images, slice(0, cfg.dim))
    for k in ("dx", "ddelta", "dz", "dB", "dC"):
        e = rel_err(to_f64(g[k][torch.from_numpy(images).cuda()]), r[k])
        assert e <= _tol(dt, k), (k, e)
    chans = np.unique(np.concatenate([[0, cfg.dim - 1], rng.choice(np.arange(1, cfg.dim - 1), 22, replace=False)]))
    r = ref(slice(0, cfg.batch), chans)
    ci = torch.from_numpy(chans).cuda()
    for k in ("dA", "dD", "ddelta_bias"):
        e = rel_err(to_f64(g[k][:, ci]), r[k])
        assert e <= _tol(dt, k), (k, e)
