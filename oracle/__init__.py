"""CPU oracle for the SS2D path: TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 implementations of what the GPU path computes, written from
the method's definitions so that a reader can check them against the pages by
eye.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from here; the product package never does,
and the two share no code.

Functions (see ``oracle/ss2d_oracle.py`` for the citations):
  cross_scan, cross_merge        exact index permutations (numpy)
  ss_fwd, ss_bwd                 the selective scan and its exact gradient (C, fp64)
  ss2d_fwd, ss2d_bwd             cross-scan -> selective scan -> cross-merge (+ gate)
  vim_bidir_fwd, vim_bidir_bwd   Vision Mamba's two-direction scan (oracle/vim_oracle.py)
  ss_step                        one recurrent step from a carried state (oracle/step_oracle.py)
  dwconv, ss2d_front_fwd/_bwd    SS2D after a depthwise conv + SiLU front (oracle/front_oracle.py)
  channel_layer_norm(_bwd),      SS2D followed by LayerNorm over channels and the gate
  ss2d_ln_fwd/_bwd                 (oracle/vss_oracle.py)
  route_projections,             SS2D with its delta/B/C produced by per-route x_proj and
  ss2d_proj_fwd/_bwd               dt_proj of the scanned sequence (oracle/proj_oracle.py)

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
closed forms, invariants, a brute-force semiseparable-matrix formulation and
finite differences; none of them is "parity unpinned".
"""
from .ss2d_oracle import (  # noqa: F401
    build_oracle_lib,
    cross_merge,
    cross_scan,
    perm_indices,
    set_num_threads,
    softplus,
    ss2d_bwd,
    ss2d_fwd,
    ss_bwd,
    ss_fwd,
)
from .front_oracle import dwconv, front_bwd, front_fwd, ss2d_front_bwd, ss2d_front_fwd  # noqa: F401
from .proj_oracle import route_projections, ss2d_proj_bwd, ss2d_proj_fwd  # noqa: F401
from .step_oracle import ss_step  # noqa: F401
from .vim_oracle import vim_bidir_bwd, vim_bidir_fwd  # noqa: F401
from .vss_oracle import channel_layer_norm, channel_layer_norm_bwd, ss2d_ln_bwd, ss2d_ln_fwd  # noqa: F401
