"""Float64 CPU oracle for exact attention (forward and backward).

TEST INFRASTRUCTURE ONLY: imported by tests, by ``__graft_entry__.smoke()`` and
by the benchmark's CPU-baseline leg, never by the product path.  It shares no
code with the HIP kernels.
"""
from .attention_fp64 import (  # noqa: F401
    as_f64, backward, dkdv_rows, dq_rows, forward, forward_rows, keep_mask,
    kv_head_index, naive_forward, score_grad_matrix,
)
