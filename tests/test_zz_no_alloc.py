"""fa_bwd_noalloc (the backward with its scratch in a static device array) against
fa_bwd_ex on the separate dQ path, through the C ABI: two calls in a row, the
second with a smaller problem, each compared with the workspace entry point's
output on the same inputs.  Both run the same kernels, so the results must agree
to the parity bound (they are expected to agree bit for bit)."""
import ctypes

import numpy as np
import pytest
import torch

from exact_attention_backward_fa_amd import inputs
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


def _noalloc(lib, case, d, o, lse, outs, device):
    from exact_attention_backward_fa_amd import _lib
    dq, dk, dv = outs
    return lib.fa_bwd_noalloc(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), o.data_ptr(),
                              lse.data_ptr(), d["do"].data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), case.B, case.Hq, case.Hkv, case.Nq, case.Nkv, case.d,
                              ctypes.c_float(case.scale), int(case.causal),
                              _lib.FA_DTYPE[case.torch_dtype],
                              torch.cuda.current_stream(device).cuda_stream)


def test_noalloc_matches_workspace_entry_point(device):
    import exact_attention_backward_fa_amd as fa
    from exact_attention_backward_fa_amd import _lib
    lib = _lib.load()
    # the larger problem first, then a smaller one that reuses the same scratch
    for name in ("llama_gqa_bf16_2048", "ragged_100x333_c"):
        case = inputs.case_by_name(name)
        pu.log(f"[gpu] noalloc {name}")
        d = pu.to_dev(inputs.make_inputs(case), device)
        o, lse = fa.fwd(d["q"], d["k"], d["v"], case.scale, case.causal)
        ref = fa.bwd(d["q"], d["k"], d["v"], o, lse, d["do"], case.scale, case.causal,
                     dq_mode="separate")
        outs = [torch.full_like(t, float("nan")) for t in ref]
        rc = _noalloc(lib, case, d, o, lse, outs, device)
        assert rc == 0, _lib.status_string(rc)
        torch.cuda.synchronize(device)
        for name_t, got, want in zip(("dq", "dk", "dv"), outs, ref):
            assert bool(torch.isfinite(got).all()), name_t
            err = pu.rel_err(got.double().cpu().numpy(), want.double().cpu().numpy())
            pu.log(f"  {name_t} rel err vs fa_bwd_ex {err:.2e}")
            assert err <= pu.TOL[case.dtype]
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), name_t


def test_noalloc_rejects_oversized_problem(device):
    from exact_attention_backward_fa_amd import _lib
    lib = _lib.load()
    cap = lib.fa_bwd_noalloc_max_scratch_bytes()
    assert cap == 16 << 20
    # 4 x 32 x 32768 query rows need 32 MiB of per-row scratch: rejected before any
    # launch, outputs untouched (tiny real buffers stand in; nothing reads them)
    q = torch.zeros(16, dtype=torch.bfloat16, device=device)
    out = torch.full((16,), 7.0, dtype=torch.bfloat16, device=device)
    p = q.data_ptr()
    rc = lib.fa_bwd_noalloc(p, p, p, p, p, p, out.data_ptr(), out.data_ptr(), out.data_ptr(),
                            4, 32, 8, 32768, 32768, 128, ctypes.c_float(0.088), 1, 1,
                            torch.cuda.current_stream(device).cuda_stream)
    assert rc == -10
    assert "scratch" in _lib.status_string(rc)
    torch.cuda.synchronize(device)
    assert bool((out == 7.0).all())
