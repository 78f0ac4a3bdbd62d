"""GPU parity of the bidirectional (Vision Mamba) scan, vim_bidir_fwd / vim_bidir_bwd, against
the fp64 oracle: outputs within 1e-4 relative for fp32 I/O and 2e-2 for bf16 I/O; gradients
within 1e-3 (bf16 I/O: 2e-2)."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ss
from gpu_util import TOL, TOL_GRAD, f64, grad_tol, rel_err, to_dev, to_f64
from selective_scan_amd import synth

pytestmark = pytest.mark.gpu

GRADS = ("du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz")


def _vim(batch, L, dim, N, dtype, z, seed, with_D=True, with_bias=True, dout=False):
    inp = synth.make_vim_inputs(batch, L, dim, N, dtype, has_z=z, seed_base=seed, with_dout=dout)
    rng = np.random.default_rng(seed)
    A = inp["A"] * np.float32(0.5 + rng.random((2, dim, 1)))    # decay varies per direction and channel
    Dv = inp["D"] * np.float32(0.7) + np.float32(0.1) * rng.standard_normal((2, dim)).astype(np.float32)
    dev = dict(u=to_dev(inp["u"], dtype), delta=to_dev(inp["delta"], dtype), A=to_dev(A, "f32"),
               B=to_dev(inp["B"], dtype), C=to_dev(inp["C"], dtype), D=to_dev(Dv, "f32") if with_D else None,
               delta_bias=to_dev(inp["delta_bias"], "f32") if with_bias else None,
               z=to_dev(inp["z"], dtype) if z else None)
    ref = dict(u=f64(inp["u"], dtype), delta=f64(inp["delta"], dtype), A=A.astype(np.float64),
               B=f64(inp["B"], dtype), C=f64(inp["C"], dtype), D=Dv.astype(np.float64) if with_D else None,
               delta_bias=inp["delta_bias"].astype(np.float64) if with_bias else None,
               z=f64(inp["z"], dtype) if z else None)
    if dout:
        return dev, ref, to_dev(inp["dout"], dtype), f64(inp["dout"], dtype)
    return dev, ref


FWD_CASES = [
    # batch, L, dim, N, dtype, z, D, bias
    (1, 7, 8, 4, "f32", True, True, True),
    (2, 197, 40, 16, "bf16", True, True, True),    # the Vim token count (odd L), dim not a multiple of 32
    (2, 64, 64, 16, "f32", False, True, True),     # L % 4 == 0: vector path
    (1, 1, 8, 1, "f32", True, True, True),         # one token
    (1, 300, 24, 8, "bf16", True, False, False),
    (2, 256, 96, 32, "f32", True, True, True),
    (1, 2048, 32, 16, "f32", True, True, True),    # few rows: chunked along the sequence
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[str(c) for c in FWD_CASES])
def test_vim_bidir_fwd(case):
    batch, L, dim, N, dtype, z, D, bias = case
    dev, ref = _vim(batch, L, dim, N, dtype, z, seed=40 + L + dim, with_D=D, with_bias=bias)
    out = ss.vim_bidir_fwd(**dev)
    assert rel_err(to_f64(out), oracle.vim_bidir_fwd(**ref)) <= TOL[dtype]


def test_vim_bidir_stages_equal_fused():
    dev, _ = _vim(2, 197, 40, 16, "bf16", True, seed=77)
    plan = ss.VimForwardPlan(**dev)
    fused = plan.run().clone()
    plan.out.zero_()
    for stage in (0, 1, 2):
        plan.run_stage(stage)
    torch.cuda.synchronize()
    assert torch.equal(plan.out.view(torch.int16), fused.view(torch.int16))


def test_vim_bidir_fwd_full_config_sampled():
    """Full Vim-Tiny size in the benchmark's launch configuration; oracle on sampled (batch, channel)
    rows (each takes both directions of its channel)."""
    cfg = synth.VIM_TINY
    inp = synth.make_vim_config_inputs(cfg, with_dout=False, params="general")
    dev = dict(u=to_dev(inp["u"], cfg.dtype), delta=to_dev(inp["delta"], cfg.dtype), A=to_dev(inp["A"], "f32"),
               B=to_dev(inp["B"], cfg.dtype), C=to_dev(inp["C"], cfg.dtype), D=to_dev(inp["D"], "f32"),
               delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], cfg.dtype))
    out = ss.vim_bidir_fwd(**dev)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = [(0, 0), (cfg.batch - 1, cfg.dim - 1)] + [
        (int(rng.integers(cfg.batch)), int(rng.integers(cfg.dim))) for _ in range(6)]
    for b, d in rows:
        sl = dict(u=inp["u"][b:b + 1, :, d:d + 1], delta=inp["delta"][b:b + 1, :, d:d + 1], B=inp["B"][b:b + 1],
                  C=inp["C"][b:b + 1], z=inp["z"][b:b + 1, d:d + 1])
        ref = {k: synth.storage_to_f64(v, cfg.dtype) for k, v in sl.items()}
        ref.update(A=inp["A"][:, d:d + 1].astype(np.float64), D=inp["D"][:, d:d + 1].astype(np.float64),
                   delta_bias=inp["delta_bias"][:, d:d + 1].astype(np.float64))
        r = oracle.vim_bidir_fwd(**ref)
        assert rel_err(to_f64(out[b:b + 1, d:d + 1]), r) <= TOL[cfg.dtype], (b, d)
    assert torch.isfinite(out.float()).all()


BWD_CASES = [
    # batch, L, dim, N, dtype, z, D, bias
    (2, 64, 64, 16, "f32", True, True, True),
    (1, 197, 40, 16, "f32", True, True, True),     # odd L
    (2, 33, 24, 4, "f32", False, False, True),
    (1, 1, 8, 8, "f32", True, True, False),        # one token
    (1, 1024, 32, 16, "f32", True, True, True),    # few rows: chunked
    (2, 197, 64, 16, "bf16", True, True, True),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(c) for c in BWD_CASES])
def test_vim_bidir_bwd(case):
    batch, L, dim, N, dtype, z, D, bias = case
    dev, ref, dout, dout64 = _vim(batch, L, dim, N, dtype, z, seed=90 + L + dim, with_D=D, with_bias=bias, dout=True)
    g = ss.vim_bidir_bwd(**dev, dout=dout)
    r = oracle.vim_bidir_bwd(**ref, dout=dout64)
    for k in GRADS:
        if r[k] is None:
            assert g[k] is None, k
            continue
        e = rel_err(to_f64(g[k]), r[k])
        assert e <= grad_tol(dtype, k), (k, e)


@pytest.mark.parametrize("case", [(2, 197, 40, 16, "bf16", True, True, True), (1, 1024, 32, 16, "f32", True, True, True),
                                  (2, 33, 24, 4, "f32", False, False, True)], ids=str)
def test_vim_bidir_bwd_reuses_forward_states(case):
    """A training forward (keep_states) then the backward on its workspace: the output of the plain
    forward and, bit for bit, the gradients of the backward that recomputes the forward (the
    chunked case included)."""
    batch, L, dim, N, dtype, z, D, bias = case
    dev, _, dout, _ = _vim(batch, L, dim, N, dtype, z, seed=140 + L, with_D=D, with_bias=bias, dout=True)
    ws = torch.empty(ss.vim_bidir_workspace_bytes(batch, dim, L, N, dev["u"].dtype), dtype=torch.uint8, device="cuda")
    out = ss.vim_bidir_fwd(**dev, workspace=ws, keep_states=True)
    assert torch.equal(out, ss.vim_bidir_fwd(**dev))
    g = ss.vim_bidir_bwd(**dev, dout=dout, workspace=ws, workspace_has_states=True)
    g2 = ss.vim_bidir_bwd(**dev, dout=dout)
    for k in GRADS:
        if g2[k] is None:
            assert g[k] is None, k
            continue
        assert torch.equal(g[k], g2[k]), k


def test_vim_bidir_bwd_full_config_sliced():
    """Vim-Tiny (B=128, L=197, D=384, N=16, bf16) forward+backward at full size, checked on oracle
    slices: per-element gradients of sampled (batch, channel) rows; dA, dD, ddelta_bias of a
    sampled channel from all sequences; dB, dC of a sampled sequence from all its channels."""
    cfg = synth.VIM_TINY
    inp = synth.make_vim_config_inputs(cfg, with_dout=True, params="general")
    dt = cfg.dtype
    dev = dict(u=to_dev(inp["u"], dt), delta=to_dev(inp["delta"], dt), A=to_dev(inp["A"], "f32"),
               B=to_dev(inp["B"], dt), C=to_dev(inp["C"], dt), D=to_dev(inp["D"], "f32"),
               delta_bias=to_dev(inp["delta_bias"], "f32"), z=to_dev(inp["z"], dt))
    g = ss.vim_bidir_bwd(**dev, dout=to_dev(inp["dout"], dt))
    torch.cuda.synchronize()
    f = lambda a: synth.storage_to_f64(a, dt)

    def ref(bs, ds):
        return oracle.vim_bidir_bwd(u=f(inp["u"][bs][:, :, ds]), delta=f(inp["delta"][bs][:, :, ds]),
                                    A=inp["A"][:, ds].astype(np.float64), B=f(inp["B"][bs]), C=f(inp["C"][bs]),
                                    D=inp["D"][:, ds].astype(np.float64),
                                    delta_bias=inp["delta_bias"][:, ds].astype(np.float64), z=f(inp["z"][bs][:, ds]),
                                    dout=f(inp["dout"][bs][:, ds]))

    rng = np.random.default_rng(31)
    tol = TOL["bf16"]
    for b, d in [(0, 0), (cfg.batch - 1, cfg.dim - 1), (int(rng.integers(cfg.batch)), int(rng.integers(cfg.dim)))]:
        r = ref(slice(b, b + 1), slice(d, d + 1))
        for k, gk in (("du", g["du"][b:b + 1, :, d:d + 1]), ("ddelta", g["ddelta"][b:b + 1, :, d:d + 1]),
                      ("dz", g["dz"][b:b + 1, d:d + 1])):
            assert rel_err(to_f64(gk), r[k]) <= tol, (k, b, d)
    d = int(rng.integers(cfg.dim))
    r = ref(slice(0, cfg.batch), slice(d, d + 1))
    for k, gk in (("dA", g["dA"][:, d:d + 1]), ("dD", g["dD"][:, d:d + 1]), ("ddelta_bias", g["ddelta_bias"][:, d:d + 1])):
        assert rel_err(to_f64(gk), r[k]) <= grad_tol(dt, k), (k, d)
    b = int(rng.integers(cfg.batch))
    r = ref(slice(b, b + 1), slice(0, cfg.dim))
    for k in ("dB", "dC"):
        assert rel_err(to_f64(g[k][b:b + 1]), r[k]) <= tol, (k, b)
