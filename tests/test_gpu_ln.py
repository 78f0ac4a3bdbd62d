"""GPU parity of SS2D with the VSS block's back half (LayerNorm over the channels of the merged
map, then the gate: ss2d_fwd / ss2d_bwd with layer_norm) against the fp64 oracle
(oracle.ss2d_ln_fwd / ss2d_ln_bwd): outputs within 1e-4 relative for fp32 I/O and 2e-2 for bf16
I/O, gradients within 1e-3 (bf16 I/O: 2e-2)."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ss
from gpu_util import TOL, TOL_GRAD, f64, grad_tol, rel_err, to_dev, to_f64
from selective_scan_amd import synth

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz", "dln_w", "dln_b", "dconv_w", "dconv_b")


def _case(batch, H, W, dim, N, dtype, z, affine, k, seed):
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, dtype, has_z=z, seed_base=seed, with_dout=True)
    rng = np.random.default_rng(seed)
    ln_w = (1.0 + 0.3 * rng.standard_normal(dim)).astype(np.float32) if affine else None
    ln_b = (0.2 * rng.standard_normal(dim)).astype(np.float32) if affine else None
    dev = dict(x=to_dev(inp["x"], dtype), delta=to_dev(inp["delta"], dtype), A=to_dev(inp["A"], "f32"),
               B=to_dev(inp["B"], dtype), C=to_dev(inp["C"], dtype), D=to_dev(inp["D"], "f32"),
               delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dtype) if z else None,
               layer_norm=True, ln_w=to_dev(ln_w, "f32") if affine else None,
               ln_b=to_dev(ln_b, "f32") if affine else None)
    ref = dict(x=f64(inp["x"], dtype), delta=f64(inp["delta"], dtype), A=inp["A"].astype(np.float64),
               B=f64(inp["B"], dtype), C=f64(inp["C"], dtype), D=inp["D"].astype(np.float64),
               delta_bias=inp["delta_bias"].astype(np.float64), z=f64(inp["z"], dtype) if z else None,
               ln_w=ln_w.astype(np.float64) if affine else None, ln_b=ln_b.astype(np.float64) if affine else None)
    if k:
        fp = synth.make_front_params(dim, k, seed_base=seed)
        dev.update(conv_w=to_dev(fp["conv_w"], "f32"), conv_b=to_dev(fp["conv_b"], "f32"))
        ref.update(conv_w=fp["conv_w"].astype(np.float64), conv_b=fp["conv_b"].astype(np.float64))
    return dev, ref, to_dev(inp["dout"], dtype), f64(inp["dout"], dtype)


CASES = [
    # batch, H, W, dim, N, dtype, z, LN scale and shift, front filter size (0: none)
    (1, 8, 8, 16, 4, "f32", True, True, 0),
    (2, 7, 9, 20, 16, "f32", True, True, 0),      # 63 pixels: one partial pixel block per image
    (1, 3, 40, 64, 8, "bf16", True, True, 0),
    (2, 14, 14, 70, 16, "bf16", False, False, 0),  # no gate, no affine: the plain normalised map
    (1, 1, 1, 8, 4, "f32", True, True, 0),         # one pixel
    (3, 5, 29, 5, 4, "f32", True, True, 0),        # fewer channels than wavefronts x 2, odd sizes
    (2, 9, 11, 24, 16, "bf16", True, True, 3),     # with the input front
    (1, 64, 64, 64, 16, "f32", True, True, 0),     # few rows: chunked route scans
    (1, 130, 72, 8, 4, "bf16", True, True, 5),     # the front's tile path
    (1, 4, 6, 300, 4, "f32", True, True, 0),       # more than 256 channels: the map is read twice
    (2, 5, 7, 260, 4, "bf16", True, False, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_ss2d_ln_fwd(case):
    batch, H, W, dim, N, dtype, z, affine, k = case
    dev, ref, _, _ = _case(batch, H, W, dim, N, dtype, z, affine, k, seed=1100 + H * W + dim)
    out = ss.ss2d_fwd(**dev)
    e = rel_err(to_f64(out), oracle.ss2d_ln_fwd(**ref))
    assert e <= TOL[dtype], e


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_ss2d_ln_bwd(case):
    batch, H, W, dim, N, dtype, z, affine, k = case
    dev, ref, dout, dout64 = _case(batch, H, W, dim, N, dtype, z, affine, k, seed=1200 + H * W + dim)
    g = ss.ss2d_bwd(**dev, dout=dout)
    r = oracle.ss2d_ln_bwd(**ref, dout=dout64)
    for key in GRADS:
        if key not in r:
            assert key not in g, key
            continue
        if r[key] is None:
            assert g.get(key) is None, key
            continue
        e = rel_err(to_f64(g[key]), r[key])
        assert e <= grad_tol(dtype, key), (key, e)


@pytest.mark.parametrize("case", [CASES[1], CASES[2], CASES[6]], ids=str)
def test_ss2d_ln_training_path(case):
    """Forward with keep_states, then the backward on its workspace: bit for bit what the
    backward that recomputes the forward gives."""
    batch, H, W, dim, N, dtype, z, affine, k = case
    dev, _, dout, _ = _case(batch, H, W, dim, N, dtype, z, affine, k, seed=1300 + H * W)
    ws = torch.empty(ss.ss2d_workspace_bytes(batch, dim, H, W, N, dev["x"].dtype), dtype=torch.uint8, device="cuda")
    out = ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
    g = ss.ss2d_bwd(**dev, dout=dout, workspace=ws, workspace_has_states=True)
    g2 = ss.ss2d_bwd(**dev, dout=dout)
    assert torch.equal(out, ss.ss2d_fwd(**dev))
    for key, v in g2.items():
        if v is None:
            assert g[key] is None
            continue
        assert torch.equal(g[key], v), key


def test_ss2d_ln_eps_matters():
    """A map with tiny per-pixel variance: the result depends on eps as the oracle's does."""
    dev, ref, _, _ = _case(1, 6, 6, 16, 4, "f32", True, True, 0, seed=1400)
    dev["x"].mul_(1e-3)
    ref["x"] = ref["x"] * 1e-3
    dev["delta"].fill_(-30.0)  # softplus ~ 0: the scan adds almost nothing; the skip term dominates
    ref["delta"] = np.full_like(ref["delta"], -30.0)
    for eps in (1e-5, 1e-2):
        out = ss.ss2d_fwd(**dev, ln_eps=eps)
        assert rel_err(to_f64(out), oracle.ss2d_ln_fwd(**ref, ln_eps=eps)) <= TOL["f32"], eps


def test_ss2d_ln_stage1_full_size_image_slices():
    """Stage-1 (B=128, 56x56, D=192, N=16, bf16) with the LayerNorm and the gate at full size,
    training launch configuration.  The normalisation couples the channels of a pixel, so the
    oracle checks whole images: the output and dx, ddelta, dz, dB, dC of sampled images."""
    cfg = synth.STAGE1
    inp = synth.make_config_inputs(cfg, with_dout=True, params="general")
    dt = cfg.dtype
    rng = np.random.default_rng(41)
    ln_w = (1.0 + 0.3 * rng.standard_normal(cfg.dim)).astype(np.float32)
    ln_b = (0.2 * rng.standard_normal(cfg.dim)).astype(np.float32)
    dev = dict(x=to_dev(inp["x"], dt), delta=to_dev(inp["delta"], dt), A=to_dev(inp["A"], "f32"),
               B=to_dev(inp["B"], dt), C=to_dev(inp["C"], dt), D=to_dev(inp["D"], "f32"),
               delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dt), layer_norm=True,
               ln_w=to_dev(ln_w, "f32"), ln_b=to_dev(ln_b, "f32"))
    ws = torch.empty(ss.ss2d_workspace_bytes(cfg.batch, cfg.dim, cfg.height, cfg.width, cfg.dstate, dev["x"].dtype),
                     dtype=torch.uint8, device="cuda")
    out = ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
    g = ss.ss2d_bwd(**dev, dout=to_dev(inp["dout"], dt), workspace=ws, workspace_has_states=True)
    torch.cuda.synchronize()
    f = lambda a: synth.storage_to_f64(a, dt)
    tol = TOL["bf16"]
    for b in (0, cfg.batch - 1, int(rng.integers(cfg.batch))):
        s = slice(b, b + 1)
        a = dict(x=f(inp["x"][s]), delta=f(inp["delta"][s]), A=inp["A"].astype(np.float64), B=f(inp["B"][s]),
                 C=f(inp["C"][s]), D=inp["D"].astype(np.float64), delta_bias=inp["delta_bias"].astype(np.float64),
                 z=f(inp["z"][s]), ln_w=ln_w.astype(np.float64), ln_b=ln_b.astype(np.float64))
        assert rel_err(to_f64(out[s]), oracle.ss2d_ln_fwd(**a)) <= tol, ("out", b)
        r = oracle.ss2d_ln_bwd(**a, dout=f(inp["dout"][s]))
        for key in ("dx", "ddelta", "dz", "dB", "dC"):
            e = rel_err(to_f64(g[key][s]), r[key])
            assert e <= tol, (key, b, e)
