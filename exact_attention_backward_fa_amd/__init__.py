"""Exact softmax attention forward and backward for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``libfa_mi355x.so`` (declared in ``include/fa_mi355x.h``); this package is the thin
Python binding over it plus the seeded workload generator used by the tests and the
benchmark.  The library is loaded on first use and there is no CPU fallback.
"""
from ._lib import (  # noqa: F401
    DQ_MODES, EXPORTS, HipEvent, auto_dq_mode, bwd, bwd_bias_dropout, bwd_into, bwd_workspace_bytes,
    fwd, fwd_bias_dropout, fwd_into, load, status_string,
)
from .autograd import attention  # noqa: F401

__all__ = ["attention", "fwd", "fwd_into", "bwd", "bwd_into", "bwd_workspace_bytes", "auto_dq_mode",
           "fwd_bias_dropout", "bwd_bias_dropout",
           "status_string", "load", "HipEvent", "DQ_MODES", "EXPORTS"]
