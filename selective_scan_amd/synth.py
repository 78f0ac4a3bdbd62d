"""Seeded synthetic inputs for the SS2D path (shared by tests and the benchmark).

This module only draws numbers and converts storage formats; it holds none of
the method's arithmetic.  The distributions copy the initialisation the pages
describe for a Mamba/VMamba layer (freeymw.com page, section 2, class `Mamba`):
  * A[k, d, n] = -(n + 1)            (S4D-real initialisation, A = -exp(A_log))
  * D[k, d] = 1
  * delta_bias = inverse-softplus of a draw in [1e-3, 1e-1]  (dt initialisation)
  * x, z, delta_raw, B, C, dout ~ N(0, 1)
Seeds: numpy PCG64 with seed = 1000 * config_index + tensor_index, tensor index in
the order x, z, delta_raw, B, C, U, dout.  Values are drawn in fp32; bf16 storage
is the round-to-nearest-even bf16 of that fp32 value, so the GPU and the oracle see
identical numbers.

The workloads use the initialisation above (params="s4d").  Parity tests draw the
parameters with no structure instead (params="general", the default of the make_*_inputs
functions): A is learned (A_log is a trained parameter of the `Mamba` module), so a kernel
must read A[k, d, n] and D[k, d] of every route, channel and state.  Then
  * A[..., n] = -exp(U[log 1/16, log 16])  per (route, channel, state), independent draws
  * D[...]    = N(1, 0.3^2)               per (route, channel)
from their own seed (tensor index T_GEN).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

T_X, T_Z, T_DELTA, T_B, T_C, T_U, T_DOUT, T_CONV, T_LN, T_PROJ, T_GEN = range(11)
PARAMS = ("s4d", "general")


@dataclass(frozen=True)
class SS2DConfig:
    name: str
    batch: int
    height: int
    width: int
    dim: int
    dstate: int
    dtype: str  # "f32" | "bf16"
    has_z: bool
    index: int  # seed base: seed = 1000 * index + tensor index
    with_bwd: bool = False

    @property
    def seqlen(self) -> int:
        return self.height * self.width

    @property
    def elements(self) -> int:
        """B*K*D*L, the unit the throughput metric counts."""
        return self.batch * 4 * self.dim * self.seqlen


# The five workloads: VMamba stage grids at 224^2 input (56^2 stage 1, 14^2 stage 3),
# channels D = 2 x embedding dim (96/192/384/768), d_state 16, and the stage-1 grid of
# a 512^2 segmentation input (128^2).
WORKLOADS = [
    SS2DConfig("tiny_8x8_d16_n4_f32", 1, 8, 8, 16, 4, "f32", True, 0),
    SS2DConfig("stage1_56x56_b128_d192_n16_bf16", 128, 56, 56, 192, 16, "bf16", True, 1),
    SS2DConfig("stage3_14x14_b128_d768_n16_bf16", 128, 14, 14, 768, 16, "bf16", True, 2),
    SS2DConfig("lowstate_56x56_b128_d96_n1_bf16_noz", 128, 56, 56, 96, 1, "bf16", False, 3),
    SS2DConfig("highres_128x128_b4_d192_n16_f32", 4, 128, 128, 192, 16, "f32", True, 4, True),
]
TINY, STAGE1, STAGE3, LOWSTATE, HIGHRES = WORKLOADS


@dataclass(frozen=True)
class VimConfig:
    """A bidirectional (Vision Mamba) workload: two scan directions over one token sequence."""
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    dtype: str
    has_z: bool
    index: int
    with_bwd: bool = False
    kind: str = "vim"

    @property
    def elements(self) -> int:
        """B*K*D*L with K = 2 directions."""
        return self.batch * 2 * self.dim * self.seqlen


# Vim-Tiny at 224^2: 14 x 14 patches of 16^2 plus the class token (L = 197), embedding 192,
# expand 2 (D = 384), d_state 16, batch 128.
VIM_WORKLOADS = [
    VimConfig("vim_tiny_l197_b128_d384_n16_bf16", 128, 197, 384, 16, "bf16", True, 5, True),
]
(VIM_TINY,) = VIM_WORKLOADS


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((bits >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored values (fp32 array or bf16 bit patterns) to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _normal(seed: int, shape, dtype: str) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def _a_d(seed_base: int, lead: tuple, dstate: int, params: str):
    """(A, D) of shapes lead + (dstate,) and lead, fp32: the S4D-real initialisation or, with
    params="general", independent draws per (route, channel[, state])."""
    if params == "s4d":
        A = np.broadcast_to(-(np.arange(dstate, dtype=np.float32) + 1.0), lead + (dstate,)).copy()
        return A, np.ones(lead, dtype=np.float32)
    if params != "general":
        raise ValueError(f"params must be one of {PARAMS}")
    rng = np.random.Generator(np.random.PCG64(1000 * seed_base + T_GEN))
    A = -np.exp(rng.uniform(np.log(1.0 / 16.0), np.log(16.0), size=lead + (dstate,))).astype(np.float32)
    D = (1.0 + 0.3 * rng.standard_normal(size=lead)).astype(np.float32)
    return A, D


def make_ss2d_inputs(batch: int, height: int, width: int, dim: int, dstate: int, dtype: str,
                     has_z: bool = True, seed_base: int = 0, with_dout: bool = False,
                     params: str = "general") -> dict:
    """Inputs of one SS2D call.  Shapes (all dense, last index fastest):
       x, z, dout: (batch, dim, H, W)      grid layout
       delta:      (batch, 4, dim, L)      per-route sequence order
       B, C:       (batch, 4, dstate, L)   per-route sequence order
       A:          (4, dim, dstate) fp32;  D, delta_bias: (4, dim) fp32
    I/O tensors are fp32 arrays or bf16 bit patterns (uint16)."""
    L = height * width
    s = 1000 * seed_base
    out = {
        "x": _normal(s + T_X, (batch, dim, height, width), dtype),
        "z": _normal(s + T_Z, (batch, dim, height, width), dtype) if has_z else None,
        "delta": _normal(s + T_DELTA, (batch, 4, dim, L), dtype),
        "B": _normal(s + T_B, (batch, 4, dstate, L), dtype),
        "C": _normal(s + T_C, (batch, 4, dstate, L), dtype),
    }
    rng = np.random.Generator(np.random.PCG64(s + T_U))
    dt = rng.uniform(1e-3, 1e-1, size=(4, dim))
    out["delta_bias"] = np.log(np.expm1(dt)).astype(np.float32)  # inverse softplus of dt
    out["A"], out["D"] = _a_d(seed_base, (4, dim), dstate, params)
    out["dout"] = _normal(s + T_DOUT, (batch, dim, height, width), dtype) if with_dout else None
    out["meta"] = dict(batch=batch, height=height, width=width, dim=dim, dstate=dstate, dtype=dtype)
    return out


def make_front_params(dim: int, k: int, seed_base: int = 0, with_bias: bool = True) -> dict:
    """Parameters of the SS2D input front: conv_w (dim, k, k) fp32 drawn N(0, 1/k^2) (unit
    gain for a unit-variance input), conv_b (dim,) fp32 drawn N(0, 0.1^2), or None."""
    rng = np.random.Generator(np.random.PCG64(1000 * seed_base + T_CONV))
    w = (rng.standard_normal(size=(dim, k, k), dtype=np.float32) / np.float32(k)).astype(np.float32)
    b = (np.float32(0.1) * rng.standard_normal(size=(dim,), dtype=np.float32)) if with_bias else None
    return {"conv_w": w, "conv_b": b}


def make_ln_params(dim: int, seed_base: int = 0) -> dict:
    """LayerNorm parameters of the VSS block's back half: ln_w = 1 + N(0, 0.3^2), ln_b = N(0, 0.2^2),
    fp32 (dim,)."""
    rng = np.random.Generator(np.random.PCG64(1000 * seed_base + T_LN))
    w = (1.0 + 0.3 * rng.standard_normal(size=(dim,), dtype=np.float32)).astype(np.float32)
    b = (np.float32(0.2) * rng.standard_normal(size=(dim,), dtype=np.float32)).astype(np.float32)
    return {"ln_w": w, "ln_b": b}


def make_proj_params(dim: int, dstate: int, dt_rank: int, seed_base: int = 0) -> dict:
    """Weights of the Δ/B/C producer, fp32: x_proj_w (4, R + 2N, dim) ~ N(0, 1/dim) (unit-variance
    projections of a unit-variance input), dt_proj_w (4, dim, R) ~ U(-R^-1/2, R^-1/2) (the `Mamba`
    module's "random" dt initialisation with dt_scale 1)."""
    rng = np.random.Generator(np.random.PCG64(1000 * seed_base + T_PROJ))
    wx = (rng.standard_normal(size=(4, dt_rank + 2 * dstate, dim), dtype=np.float32) / np.float32(np.sqrt(dim)))
    std = np.float32(dt_rank ** -0.5)
    wdt = rng.uniform(-std, std, size=(4, dim, dt_rank)).astype(np.float32)
    return {"x_proj_w": wx.astype(np.float32), "dt_proj_w": wdt}


def make_config_inputs(cfg: SS2DConfig, with_dout: bool | None = None, params: str = "s4d") -> dict:
    """Inputs of a workload: its parameters as the workload states them (params="s4d") unless
    a test asks for general ones."""
    return make_ss2d_inputs(cfg.batch, cfg.height, cfg.width, cfg.dim, cfg.dstate, cfg.dtype,
                            cfg.has_z, cfg.index, cfg.with_bwd if with_dout is None else with_dout, params)


def make_ss_inputs(batch: int, dim: int, dstate: int, seqlen: int, ngroups: int, dtype: str,
                   has_z: bool = True, seed_base: int = 0, with_dout: bool = False,
                   params: str = "general") -> dict:
    """Inputs of one generic selective-scan call (the `selective_scan_fn` shapes):
       u, delta, z, dout: (batch, dim, L); B, C: (batch, G, N, L); A: (dim, N) fp32;
       D, delta_bias: (dim,) fp32."""
    s = 1000 * seed_base
    out = {
        "u": _normal(s + T_X, (batch, dim, seqlen), dtype),
        "z": _normal(s + T_Z, (batch, dim, seqlen), dtype) if has_z else None,
        "delta": _normal(s + T_DELTA, (batch, dim, seqlen), dtype),
        "B": _normal(s + T_B, (batch, ngroups, dstate, seqlen), dtype),
        "C": _normal(s + T_C, (batch, ngroups, dstate, seqlen), dtype),
    }
    rng = np.random.Generator(np.random.PCG64(s + T_U))
    dt = rng.uniform(1e-3, 1e-1, size=(dim,))
    out["delta_bias"] = np.log(np.expm1(dt)).astype(np.float32)
    out["A"], out["D"] = _a_d(seed_base, (dim,), dstate, params)
    out["dout"] = _normal(s + T_DOUT, (batch, dim, seqlen), dtype) if with_dout else None
    out["meta"] = dict(batch=batch, dim=dim, dstate=dstate, seqlen=seqlen, ngroups=ngroups, dtype=dtype)
    return out


def make_vim_inputs(batch: int, seqlen: int, dim: int, dstate: int, dtype: str, has_z: bool = True,
                    seed_base: int = 0, with_dout: bool = False, params: str = "general") -> dict:
    """Inputs of one bidirectional scan call.  Shapes (dense, last index fastest):
       u, delta:  (batch, 2, dim, L)      direction k in its own scan order
       B, C:      (batch, 2, dstate, L)   direction k in its own scan order
       z, dout:   (batch, dim, L)         forward order
       A:         (2, dim, dstate) fp32;  D, delta_bias: (2, dim) fp32
    Draws as for SS2D (u takes the x slot of the seed table)."""
    s = 1000 * seed_base
    out = {
        "u": _normal(s + T_X, (batch, 2, dim, seqlen), dtype),
        "z": _normal(s + T_Z, (batch, dim, seqlen), dtype) if has_z else None,
        "delta": _normal(s + T_DELTA, (batch, 2, dim, seqlen), dtype),
        "B": _normal(s + T_B, (batch, 2, dstate, seqlen), dtype),
        "C": _normal(s + T_C, (batch, 2, dstate, seqlen), dtype),
    }
    rng = np.random.Generator(np.random.PCG64(s + T_U))
    dt = rng.uniform(1e-3, 1e-1, size=(2, dim))
    out["delta_bias"] = np.log(np.expm1(dt)).astype(np.float32)
    out["A"], out["D"] = _a_d(seed_base, (2, dim), dstate, params)
    out["dout"] = _normal(s + T_DOUT, (batch, dim, seqlen), dtype) if with_dout else None
    out["meta"] = dict(batch=batch, seqlen=seqlen, dim=dim, dstate=dstate, dtype=dtype)
    return out


def make_vim_config_inputs(cfg: VimConfig, with_dout: bool | None = None, params: str = "s4d") -> dict:
    return make_vim_inputs(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, cfg.dtype, cfg.has_z, cfg.index,
                           cfg.with_bwd if with_dout is None else with_dout, params)
