"""Helpers shared by the GPU parity tests (moving seeded numpy inputs to the device and back,
and the relative-error measure the tolerances are stated in)."""
import numpy as np
import torch

from selective_scan_amd import synth

# Tolerances: max relative error, elementwise against max(|ref|, rms(ref)).
TOL = {"f32": 1e-4, "bf16": 2e-2}
TOL_GRAD = 1e-3
# Gradients that every path stores in fp32 whatever the I/O type (parameters and weights).
FP32_GRADS = frozenset({"dA", "dD", "ddelta_bias", "dconv_w", "dconv_b", "dln_w", "dln_b", "dx_proj_w",
                        "ddt_proj_w"})


def grad_tol(dtype, key):
    """1e-3 for fp32 I/O and for the gradients stored in fp32; 2e-2 for gradients stored in bf16
    (one rounding to bf16 is up to 2^-9 relative, as for a bf16 output)."""
    return TOL_GRAD if dtype == "f32" or key in FP32_GRADS else TOL["bf16"]


def to_dev(a, dtype):
    """numpy storage (fp32 array, or bf16 bit patterns as uint16) -> torch tensor on cuda:0."""
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_f64(t):
    """torch tensor (fp32 or bf16) -> numpy float64, exactly."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def f64(a, dtype):
    return None if a is None else synth.storage_to_f64(a, dtype)


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.isfinite(got).all(), "non-finite values in GPU result"
    rms = np.sqrt(np.mean(ref * ref))
    denom = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(got - ref) / denom))


def random_bits(shape, dtype, seed):
    """Random non-NaN, non-Inf bit patterns of the storage type (for bit-exact copies)."""
    rng = np.random.default_rng(seed)
    if dtype == "bf16":
        b = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
        exp = (b >> 7) & 0xFF
        b[exp == 0xFF] &= np.uint16(0xBFFF)  # clear one exponent bit: finite
        return b
    b = rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32)
    exp = (b >> 23) & 0xFF
    b[exp == 0xFF] &= np.uint32(0xBFFFFFFF)
    return b.view(np.float32)
