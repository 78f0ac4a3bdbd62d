"""GPU parity of selective_scan_step (one recurrent step from a carried state) against the fp64
oracle, and consistency of chained steps with the sequence scan's outputs and last state."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ss
from gpu_util import TOL, f64, rel_err, to_dev, to_f64
from selective_scan_amd import synth

pytestmark = pytest.mark.gpu

STEP_CASES = [
    # batch, dim, N, G, dtype, z, D, bias, softplus
    (2, 64, 16, 1, "f32", True, True, True, True),
    (3, 48, 3, 2, "f32", False, True, False, True),   # N padded to 4
    (1, 96, 64, 4, "bf16", True, True, True, True),
    (4, 10, 1, 1, "f32", True, False, True, True),
    (2, 32, 8, 1, "f32", True, True, False, False),   # no softplus
    (2, 40, 32, 2, "bf16", False, True, True, True),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[str(c) for c in STEP_CASES])
def test_selective_scan_step(case):
    batch, dim, N, G, dtype, z, D, bias, sp = case
    rng = np.random.default_rng(batch * 1000 + dim + N)
    inp = synth.make_ss_inputs(batch, dim, N, 1, G, dtype, has_z=z, seed_base=600 + dim + N)
    state0 = rng.standard_normal((batch, dim, N)).astype(np.float32)
    delta = inp["delta"][..., 0]
    if not sp:
        delta = (delta & np.uint16(0x7FFF)) if dtype == "bf16" else np.abs(delta)
    A = inp["A"] * np.float32(0.5 + rng.random((dim, 1)))
    dev = dict(x=to_dev(inp["u"][..., 0], dtype), delta=to_dev(delta, dtype), A=to_dev(A, "f32"),
               B=to_dev(inp["B"][..., 0], dtype), C=to_dev(inp["C"][..., 0], dtype),
               D=to_dev(inp["D"], "f32") if D else None, z=to_dev(inp["z"][..., 0], dtype) if z else None,
               delta_bias=to_dev(inp["delta_bias"], "f32") if bias and sp else None)
    state = torch.from_numpy(state0.copy()).cuda()
    out = ss.selective_scan_step(state, **dev, delta_softplus=sp)
    r_out, r_state = oracle.ss_step(state0.astype(np.float64), f64(inp["u"][..., 0], dtype), f64(delta, dtype),
                                    A.astype(np.float64), f64(inp["B"][..., 0], dtype), f64(inp["C"][..., 0], dtype),
                                    inp["D"].astype(np.float64) if D else None,
                                    f64(inp["z"][..., 0], dtype) if z else None,
                                    inp["delta_bias"].astype(np.float64) if bias and sp else None, sp)
    assert rel_err(to_f64(out), r_out) <= TOL[dtype]
    assert rel_err(state.cpu().numpy().astype(np.float64), r_state) <= 1e-5


def test_steps_continue_the_sequence_scan():
    """selective_scan_fwd over the first part (last_state), then steps over the rest: outputs match
    the scan of the whole sequence and the final state its last_state."""
    batch, dim, N, L, cut = 2, 64, 16, 40, 29
    inp = synth.make_ss_inputs(batch, dim, N, L, 1, "f32", has_z=True, seed_base=650)
    dev = {k: to_dev(inp[k], "f32") for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    full, last = ss.selective_scan_fwd(**dev, delta_softplus=True, return_last_state=True)
    first = {k: (v[..., :cut].contiguous() if k in ("u", "delta", "B", "C", "z") else v) for k, v in dev.items()}
    _, state = ss.selective_scan_fwd(**first, delta_softplus=True, return_last_state=True)
    for t in range(cut, L):
        out = ss.selective_scan_step(state, dev["u"][..., t].contiguous(), dev["delta"][..., t].contiguous(), dev["A"],
                                     dev["B"][..., t].contiguous(), dev["C"][..., t].contiguous(), dev["D"],
                                     z=dev["z"][..., t].contiguous(), delta_bias=dev["delta_bias"],
                                     delta_softplus=True)
        assert rel_err(to_f64(out), to_f64(full[..., t])) <= 1e-5, t
    assert rel_err(to_f64(state), to_f64(last)) <= 1e-5
