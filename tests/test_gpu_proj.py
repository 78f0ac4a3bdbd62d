"""GPU parity of SS2D with its Δ/B/C producer (per-route x_proj and dt_proj of the scanned sequence
on the matrix cores, then fp32 route scans: ss2d_fwd / ss2d_bwd with x_proj_w, dt_proj_w) against
the fp64 oracle (oracle.ss2d_proj_fwd / ss2d_proj_bwd): outputs within 1e-4 relative for fp32 I/O
and 2e-2 for bf16 I/O, gradients within 1e-3 (bf16 I/O: 2e-2)."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ss
from gpu_util import TOL, TOL_GRAD, f64, grad_tol, rel_err, to_dev, to_f64
from selective_scan_amd import synth

pytestmark = pytest.mark.gpu

GRADS = ("dx", "dx_proj_w", "ddt_proj_w", "dA", "dD", "ddelta_bias", "dz", "dln_w", "dln_b", "dconv_w", "dconv_b")


def _case(batch, H, W, dim, N, R, dtype, z, k, ln, seed):
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, dtype, has_z=z, seed_base=seed, with_dout=True)
    pw = synth.make_proj_params(dim, N, R, seed_base=seed)
    dev = dict(x=to_dev(inp["x"], dtype), delta=None, A=to_dev(inp["A"], "f32"), B=None, C=None,
               D=to_dev(inp["D"], "f32"), delta_bias=to_dev(inp["delta_bias"], "f32"),
               z=to_dev(inp["z"], dtype) if z else None,
               x_proj_w=to_dev(pw["x_proj_w"], "f32"), dt_proj_w=to_dev(pw["dt_proj_w"], "f32"))
    ref = dict(x=f64(inp["x"], dtype), x_proj_w=pw["x_proj_w"].astype(np.float64),
               dt_proj_w=pw["dt_proj_w"].astype(np.float64), A=inp["A"].astype(np.float64),
               D=inp["D"].astype(np.float64), delta_bias=inp["delta_bias"].astype(np.float64),
               z=f64(inp["z"], dtype) if z else None)
    if k:
        fp = synth.make_front_params(dim, k, seed_base=seed)
        dev.update(conv_w=to_dev(fp["conv_w"], "f32"), conv_b=to_dev(fp["conv_b"], "f32"))
        ref.update(conv_w=fp["conv_w"].astype(np.float64), conv_b=fp["conv_b"].astype(np.float64))
    if ln:
        lp = synth.make_ln_params(dim, seed_base=seed)
        dev.update(layer_norm=True, ln_w=to_dev(lp["ln_w"], "f32"), ln_b=to_dev(lp["ln_b"], "f32"))
        ref.update(layer_norm=True, ln_w=lp["ln_w"].astype(np.float64), ln_b=lp["ln_b"].astype(np.float64))
    return dev, ref, to_dev(inp["dout"], dtype), f64(inp["dout"], dtype)


CASES = [
    # batch, H, W, dim, N, dt_rank, dtype, z, front filter (0: none), LayerNorm
    (1, 8, 8, 16, 4, 2, "f32", True, 0, False),
    (2, 7, 9, 20, 16, 3, "f32", True, 0, False),      # ragged GEMM tiles (L = 63)
    (1, 3, 40, 64, 8, 4, "bf16", True, 0, False),
    (2, 14, 14, 70, 16, 5, "bf16", False, 3, True),   # with the front and the LayerNorm, no gate
    (1, 1, 1, 8, 4, 1, "f32", True, 0, False),        # one pixel
    (1, 64, 64, 64, 16, 4, "f32", True, 0, False),    # few rows: chunked route scans
    (2, 9, 11, 96, 16, 6, "bf16", True, 3, True),     # dim over one 64-row tile
    (3, 5, 6, 24, 1, 2, "f32", True, 0, False),       # one state
    (1, 10, 12, 48, 8, 12, "f32", True, 0, False),    # rank 9..16: the wider in-scan dt_proj
    (1, 5, 7, 32, 16, 9, "bf16", True, 0, False),     # same, L % 4 != 0 (scalar loads)
    (2, 6, 8, 40, 4, 20, "bf16", True, 3, False),     # rank > 16: delta through its own product
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_ss2d_proj_fwd(case):
    batch, H, W, dim, N, R, dtype, z, k, ln = case
    dev, ref, _, _ = _case(batch, H, W, dim, N, R, dtype, z, k, ln, seed=1600 + H * W + dim)
    out = ss.ss2d_fwd(**dev)
    e = rel_err(to_f64(out), oracle.ss2d_proj_fwd(**ref))
    assert e <= TOL[dtype], e


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_ss2d_proj_bwd(case):
    batch, H, W, dim, N, R, dtype, z, k, ln = case
    dev, ref, dout, dout64 = _case(batch, H, W, dim, N, R, dtype, z, k, ln, seed=1700 + H * W + dim)
    g = ss.ss2d_bwd(**dev, dout=dout)
    r = oracle.ss2d_proj_bwd(**ref, dout=dout64)
    assert g["ddelta"] is None and g["dB"] is None and g["dC"] is None
    for key in GRADS:
        if r.get(key) is None:
            assert g.get(key) is None, key
            continue
        e = rel_err(to_f64(g[key]), r[key])
        assert e <= grad_tol(dtype, key), (key, e)


@pytest.mark.parametrize("case", [CASES[1], CASES[3]], ids=str)
def test_ss2d_proj_training_path(case):
    """Forward with keep_states, then the backward on its workspace: bit for bit what the
    backward that recomputes the projections and the forward gives."""
    batch, H, W, dim, N, R, dtype, z, k, ln = case
    dev, _, dout, _ = _case(batch, H, W, dim, N, R, dtype, z, k, ln, seed=1800 + H * W)
    ws = torch.empty(ss.ss2d_workspace_bytes(batch, dim, H, W, N, dev["x"].dtype, R), dtype=torch.uint8,
                     device="cuda")
    out = ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
    g = ss.ss2d_bwd(**dev, dout=dout, workspace=ws, workspace_has_states=True)
    g2 = ss.ss2d_bwd(**dev, dout=dout)
    assert torch.equal(out, ss.ss2d_fwd(**dev))
    for key, v in g2.items():
        if v is None:
            assert g[key] is None
            continue
        assert torch.equal(g[key], v), key


def test_ss2d_proj_stage1_full_size_image_slices():
    """Stage-1 (B=128, 56x56, D=192, N=16, dt_rank 6, bf16) with the producer, the 3x3 front and the
    LayerNorm at full size, training launch configuration.  The projections mix a pixel's channels,
    so the oracle checks whole images: the output, dx and dz of sampled images."""
    cfg = synth.STAGE1
    inp = synth.make_config_inputs(cfg, with_dout=True, params="general")
    R = 6
    pw = synth.make_proj_params(cfg.dim, cfg.dstate, R, seed_base=cfg.index)
    fp = synth.make_front_params(cfg.dim, 3, seed_base=cfg.index)
    lp = synth.make_ln_params(cfg.dim, seed_base=cfg.index)
    dt = cfg.dtype
    dev = dict(x=to_dev(inp["x"], dt), delta=None, A=to_dev(inp["A"], "f32"), B=None, C=None,
               D=to_dev(inp["D"], "f32"), delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dt),
               x_proj_w=to_dev(pw["x_proj_w"], "f32"), dt_proj_w=to_dev(pw["dt_proj_w"], "f32"),
               conv_w=to_dev(fp["conv_w"], "f32"), conv_b=to_dev(fp["conv_b"], "f32"), layer_norm=True,
               ln_w=to_dev(lp["ln_w"], "f32"), ln_b=to_dev(lp["ln_b"], "f32"))
    ws = torch.empty(ss.ss2d_workspace_bytes(cfg.batch, cfg.dim, cfg.height, cfg.width, cfg.dstate,
                                             dev["x"].dtype, R), dtype=torch.uint8, device="cuda")
    out = ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
    g = ss.ss2d_bwd(**dev, dout=to_dev(inp["dout"], dt), workspace=ws, workspace_has_states=True)
    torch.cuda.synchronize()
    f = lambda a: synth.storage_to_f64(a, dt)
    tol = TOL["bf16"]
    rng = np.random.default_rng(51)
    for b in (0, int(rng.integers(cfg.batch))):
        s = slice(b, b + 1)
        a = dict(x=f(inp["x"][s]), x_proj_w=pw["x_proj_w"].astype(np.float64),
                 dt_proj_w=pw["dt_proj_w"].astype(np.float64), A=inp["A"].astype(np.float64),
                 D=inp["D"].astype(np.float64), delta_bias=inp["delta_bias"].astype(np.float64), z=f(inp["z"][s]),
                 conv_w=fp["conv_w"].astype(np.float64), conv_b=fp["conv_b"].astype(np.float64), layer_norm=True,
                 ln_w=lp["ln_w"].astype(np.float64), ln_b=lp["ln_b"].astype(np.float64))
        assert rel_err(to_f64(out[s]), oracle.ss2d_proj_fwd(**a)) <= tol, ("out", b)
        r = oracle.ss2d_proj_bwd(**a, dout=f(inp["dout"][s]))
        for key in ("dx", "dz"):
            e = rel_err(to_f64(g[key][s]), r[key])
            assert e <= tol, (key, b, e)
    assert all(torch.isfinite(g[k]).all() for k in ("dx_proj_w", "ddt_proj_w", "dA", "dconv_w", "dln_w"))


def test_ss2d_proj_stage3_full_size_rank24():
    """Stage-3 (B=128, 14x14, D=768, N=16, bf16) with the producer at dt_rank 24 (delta through
    its own product), training launch configuration: the output, dx and dz of sampled images
    against the oracle; the weight gradients, sums over all images, equal the sums of those of
    the two half batches (whose slices group the images' steps differently), to fp32 rounding."""
    cfg = synth.STAGE3
    inp = synth.make_config_inputs(cfg, with_dout=True, params="general")
    R = 24
    pw = synth.make_proj_params(cfg.dim, cfg.dstate, R, seed_base=cfg.index)
    dt = cfg.dtype

    def run(sl):
        dev = dict(x=to_dev(inp["x"][sl], dt), delta=None, A=to_dev(inp["A"], "f32"), B=None, C=None,
                   D=to_dev(inp["D"], "f32"), delta_bias=to_dev(inp["delta_bias"], "f32"),
                   z=to_dev(inp["z"][sl], dt), x_proj_w=to_dev(pw["x_proj_w"], "f32"),
                   dt_proj_w=to_dev(pw["dt_proj_w"], "f32"))
        nb = dev["x"].shape[0]
        ws = torch.empty(ss.ss2d_workspace_bytes(nb, cfg.dim, cfg.height, cfg.width, cfg.dstate, dev["x"].dtype, R),
                         dtype=torch.uint8, device="cuda")
        out = ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
        g = ss.ss2d_bwd(**dev, dout=to_dev(inp["dout"][sl], dt), workspace=ws, workspace_has_states=True)
        torch.cuda.synchronize()
        return out, g

    out, g = run(slice(0, cfg.batch))
    f = lambda a: synth.storage_to_f64(a, dt)
    tol = TOL["bf16"]
    rng = np.random.default_rng(53)
    for b in (cfg.batch - 1, int(rng.integers(cfg.batch))):
        s = slice(b, b + 1)
        a = dict(x=f(inp["x"][s]), x_proj_w=pw["x_proj_w"].astype(np.float64),
                 dt_proj_w=pw["dt_proj_w"].astype(np.float64), A=inp["A"].astype(np.float64),
                 D=inp["D"].astype(np.float64), delta_bias=inp["delta_bias"].astype(np.float64), z=f(inp["z"][s]))
        assert rel_err(to_f64(out[s]), oracle.ss2d_proj_fwd(**a)) <= tol, ("out", b)
        r = oracle.ss2d_proj_bwd(**a, dout=f(inp["dout"][s]))
        for key in ("dx", "dz"):
            e = rel_err(to_f64(g[key][s]), r[key])
            assert e <= tol, (key, b, e)
    h = cfg.batch // 2
    _, g1 = run(slice(0, h))
    _, g2 = run(slice(h, cfg.batch))
    for key in ("dx_proj_w", "ddt_proj_w", "dA", "dD", "ddelta_bias"):
        e = rel_err(to_f64(g[key]), to_f64(g1[key]) + to_f64(g2[key]))
        assert e <= 1e-4, (key, e)
