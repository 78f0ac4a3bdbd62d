"""GPU parity of SS2D with its input front (depthwise k x k convolution + SiLU before the
cross-scan: ss2d_fwd / ss2d_bwd with conv_w, conv_b) against the fp64 oracle
(oracle.ss2d_front_fwd / ss2d_front_bwd): outputs within 1e-4 relative for fp32 I/O and 2e-2 for
bf16 I/O, gradients within 1e-3 (bf16 I/O: 2e-2)."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ss
from gpu_util import TOL, TOL_GRAD, f64, grad_tol, rel_err, to_dev, to_f64
from selective_scan_amd import synth

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz", "dconv_w", "dconv_b")


def _case(batch, H, W, dim, N, dtype, z, k, bias, seed):
    inp = synth.make_ss2d_inputs(batch, H, W, dim, N, dtype, has_z=z, seed_base=seed, with_dout=True)
    fp = synth.make_front_params(dim, k, seed_base=seed, with_bias=bias)
    dev = dict(x=to_dev(inp["x"], dtype), delta=to_dev(inp["delta"], dtype), A=to_dev(inp["A"], "f32"),
               B=to_dev(inp["B"], dtype), C=to_dev(inp["C"], dtype), D=to_dev(inp["D"], "f32"),
               delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dtype) if z else None,
               conv_w=to_dev(fp["conv_w"], "f32"), conv_b=to_dev(fp["conv_b"], "f32") if bias else None)
    ref = dict(x=f64(inp["x"], dtype), delta=f64(inp["delta"], dtype), A=inp["A"].astype(np.float64),
               B=f64(inp["B"], dtype), C=f64(inp["C"], dtype), D=inp["D"].astype(np.float64),
               delta_bias=inp["delta_bias"].astype(np.float64), z=f64(inp["z"], dtype) if z else None,
               conv_w=fp["conv_w"].astype(np.float64), conv_b=fp["conv_b"].astype(np.float64) if bias else None)
    return dev, ref, to_dev(inp["dout"], dtype), f64(inp["dout"], dtype)


CASES = [
    # batch, H, W, dim, N, dtype, z, k, conv bias
    (1, 8, 8, 16, 4, "f32", True, 3, True),
    (2, 7, 9, 20, 16, "f32", True, 5, True),     # ragged, filter wider than the map's short side
    (1, 3, 40, 64, 8, "bf16", True, 3, False),
    (2, 33, 35, 24, 16, "f32", False, 7, True),  # 7 x 7 filter (halo 3), odd sizes
    (1, 1, 1, 8, 4, "f32", True, 3, True),       # one pixel: only the filter's centre tap sees data
    (2, 14, 14, 70, 16, "bf16", True, 1, True),  # 1 x 1 filter: a per-channel scale and shift
    (1, 64, 64, 64, 16, "f32", True, 3, True),   # few rows: chunked route scans
    # maps whose halo'd planes exceed 64 KB of LDS: the 32 x 32 tile kernels
    (1, 100, 90, 8, 4, "f32", True, 5, True),
    (1, 130, 72, 8, 4, "bf16", True, 3, False),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_ss2d_front_fwd(case):
    batch, H, W, dim, N, dtype, z, k, bias = case
    dev, ref, _, _ = _case(batch, H, W, dim, N, dtype, z, k, bias, seed=500 + H * W + k)
    out = ss.ss2d_fwd(**dev)
    assert rel_err(to_f64(out), oracle.ss2d_front_fwd(**ref)) <= TOL[dtype]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_ss2d_front_bwd(case):
    batch, H, W, dim, N, dtype, z, k, bias = case
    dev, ref, dout, dout64 = _case(batch, H, W, dim, N, dtype, z, k, bias, seed=600 + H * W + k)
    g = ss.ss2d_bwd(**dev, dout=dout)
    r = oracle.ss2d_front_bwd(**ref, dout=dout64)
    for key in GRADS:
        if r[key] is None:
            assert g[key] is None, key
            continue
        e = rel_err(to_f64(g[key]), r[key])
        assert e <= grad_tol(dtype, key), (key, e)


@pytest.mark.parametrize("case", [CASES[1], CASES[2], CASES[3]], ids=str)
def test_ss2d_front_training_path(case):
    """Forward with keep_states, then the backward on its workspace: bit for bit what the
    backward that recomputes the front and the forward gives, and the plain forward's output."""
    batch, H, W, dim, N, dtype, z, k, bias = case
    dev, _, dout, _ = _case(batch, H, W, dim, N, dtype, z, k, bias, seed=700 + H * W)
    ws = torch.empty(ss.ss2d_workspace_bytes(batch, dim, H, W, N, dev["x"].dtype), dtype=torch.uint8, device="cuda")
    out = ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
    g = ss.ss2d_bwd(**dev, dout=dout, workspace=ws, workspace_has_states=True)
    g2 = ss.ss2d_bwd(**dev, dout=dout)
    assert torch.equal(out, ss.ss2d_fwd(**dev))
    for key in GRADS:
        if g2[key] is None:
            assert g[key] is None
            continue
        assert torch.equal(g[key], g2[key]), key


def test_ss2d_front_identity_filter_equals_plain_ss2d_on_silu():
    """A centred one-hot filter without bias makes the front silu(x): the result equals plain
    ss2d_fwd on silu(x) computed in fp32 (fp32 I/O, so the stored front output is exact up to
    the silu's own rounding)."""
    dev, _, _, _ = _case(2, 9, 11, 16, 8, "f32", True, 3, False, seed=811)
    w = torch.zeros_like(dev["conv_w"])
    w[:, 1, 1] = 1.0
    out = ss.ss2d_fwd(**{**dev, "conv_w": w})
    plain = ss.ss2d_fwd(**{**dev, "conv_w": None, "x": torch.nn.functional.silu(dev["x"])})
    assert rel_err(to_f64(out), to_f64(plain)) <= 1e-6


def test_ss2d_front_stage1_full_size_sampled():
    """Stage-1 (B=128, 56x56, D=192, N=16, bf16) with a 3 x 3 front at full size, training launch
    configuration.  The front is per channel, so the oracle checks (image, channel) planes of the
    output and of dx, ddelta, dz, and one channel's filter gradients over all images."""
    cfg = synth.STAGE1
    inp = synth.make_config_inputs(cfg, with_dout=True, params="general")
    fp = synth.make_front_params(cfg.dim, 3, seed_base=cfg.index)
    dt = cfg.dtype
    dev = dict(x=to_dev(inp["x"], dt), delta=to_dev(inp["delta"], dt), A=to_dev(inp["A"], "f32"),
               B=to_dev(inp["B"], dt), C=to_dev(inp["C"], dt), D=to_dev(inp["D"], "f32"),
               delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dt),
               conv_w=to_dev(fp["conv_w"], "f32"), conv_b=to_dev(fp["conv_b"], "f32"))
    ws = torch.empty(ss.ss2d_workspace_bytes(cfg.batch, cfg.dim, cfg.height, cfg.width, cfg.dstate, dev["x"].dtype),
                     dtype=torch.uint8, device="cuda")
    out = ss.ss2d_fwd(**dev, workspace=ws, keep_states=True)
    g = ss.ss2d_bwd(**dev, dout=to_dev(inp["dout"], dt), workspace=ws, workspace_has_states=True)
    torch.cuda.synchronize()
    f = lambda a: synth.storage_to_f64(a, dt)

    def ref_args(bs, ds):
        return dict(x=f(inp["x"][bs][:, ds]), delta=f(inp["delta"][bs][:, :, ds]), A=inp["A"][:, ds].astype(np.float64),
                    B=f(inp["B"][bs]), C=f(inp["C"][bs]), D=inp["D"][:, ds].astype(np.float64),
                    delta_bias=inp["delta_bias"][:, ds].astype(np.float64), z=f(inp["z"][bs][:, ds]),
                    conv_w=fp["conv_w"][ds].astype(np.float64), conv_b=fp["conv_b"][ds].astype(np.float64))

    rng = np.random.default_rng(23)
    tol = TOL["bf16"]
    for b, d in [(0, 0), (cfg.batch - 1, cfg.dim - 1), (int(rng.integers(cfg.batch)), int(rng.integers(cfg.dim)))]:
        a = ref_args(slice(b, b + 1), slice(d, d + 1))
        assert rel_err(to_f64(out[b:b + 1, d:d + 1]), oracle.ss2d_front_fwd(**a)) <= tol, ("out", b, d)
        r = oracle.ss2d_front_bwd(**a, dout=f(inp["dout"][b:b + 1, d:d + 1]))
        for key, gk in (("dx", g["dx"][b:b + 1, d:d + 1]), ("ddelta", g["ddelta"][b:b + 1, :, d:d + 1]),
                        ("dz", g["dz"][b:b + 1, d:d + 1])):
            e = rel_err(to_f64(gk), r[key])
            assert e <= tol, (key, b, d, e)
    d = int(rng.integers(cfg.dim))
    r = oracle.ss2d_front_bwd(**ref_args(slice(0, cfg.batch), slice(d, d + 1)),
                              dout=f(inp["dout"][:, d:d + 1]))
    for key in ("dconv_w", "dconv_b", "dA", "dD", "ddelta_bias"):
        gk = g[key][d:d + 1] if key in ("dconv_w", "dconv_b") else g[key][:, d:d + 1]
        e = rel_err(to_f64(gk), r[key])
        assert e <= grad_tol(dt, key), (key, d, e)
