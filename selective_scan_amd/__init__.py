"""SS2D on AMD Instinct MI355X: cross-scan -> selective scan (S6) -> cross-merge, and the
two-direction scan of Vision Mamba.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI in
include/ss2d.h (libss2d.so, built in-tree by __graft_entry__.build()).  This package
is the thin Python binding over that ABI; its functions carry the C entry points' names.
"""
from ._binding import (  # noqa: F401
    SS2DError,
    SS2DForwardPlan,
    lib,
    selective_scan_bwd,
    selective_scan_fwd,
    selective_scan_step,
    selective_scan_workspace_bytes,
    ss2d_bwd,
    ss2d_cross_merge,
    ss2d_cross_scan,
    ss2d_fwd,
    ss2d_fwd_noalloc,
    ss2d_fwd_noalloc_max_workspace_bytes,
    ss2d_workspace_bytes,
    VimForwardPlan,
    vim_bidir_bwd,
    vim_bidir_fwd,
    vim_bidir_workspace_bytes,
)
from .autograd import SelectiveScanFn, SS2DFn, VimBidirFn, selective_scan_fn, ss2d, vim_bidir  # noqa: F401,E402
