"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run the
fp64 oracle on the same seeded inputs, and measure errors the way the gate states
them (max|g - ref| / max|ref| per tensor; LSE as max absolute error)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.attention_fp64 as orc

TOL = {"fp16": 1e-2, "bf16": 2e-2}
LSE_TOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    return num / den if den > 1e-30 else num


def lse_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    if not np.array_equal(fin, np.isfinite(got)):
        return float("inf")
    # rows with no visible key must be exactly -inf on both sides
    if not np.all(got[~fin] == ref[~fin]):
        return float("inf")
    return float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0


def to_dev(x: dict, device) -> dict:
    return {k: v.to(device) for k, v in x.items()}


def gpu_forward_backward(case, x: dict, device, dq_mode="auto", o_lse=None):
    """Run fa_fwd then fa_bwd_ex on the GPU.  With ``o_lse`` the backward is fed
    that (o, lse) pair instead of the GPU forward's.  Returns CPU tensors."""
    import exact_attention_backward_fa_amd as fa
    d = to_dev(x, device)
    o, lse = fa.fwd(d["q"], d["k"], d["v"], case.scale, case.causal)
    if o_lse is not None:
        ob, lb = o_lse[0].to(device), o_lse[1].to(device)
    else:
        ob, lb = o, lse
    dq, dk, dv = fa.bwd(d["q"], d["k"], d["v"], ob, lb, d["do"], case.scale, case.causal,
                        dq_mode=dq_mode)
    torch.cuda.synchronize(device)
    return {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}


def group_slices(case, x: dict, b: int, g: int) -> dict:
    """Inputs of one (batch, kv head) group: its G query heads and its K/V head."""
    G = case.Hq // case.Hkv
    return {
        "q": x["q"][b:b + 1, g * G:(g + 1) * G],
        "k": x["k"][b:b + 1, g:g + 1],
        "v": x["v"][b:b + 1, g:g + 1],
        "do": x["do"][b:b + 1, g * G:(g + 1) * G],
    }


def oracle_group(case, x: dict, b: int, g: int):
    """Full fp64 oracle (forward and backward) for one group."""
    s = group_slices(case, x, b, g)
    o, lse = orc.forward(s["q"], s["k"], s["v"], case.scale, case.causal)
    dq, dk, dv = orc.backward(s["q"], s["k"], s["v"], s["do"], case.scale, case.causal)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def gpu_group(case, res: dict, b: int, g: int) -> dict:
    G = case.Hq // case.Hkv
    out = {}
    for key in ("o", "dq"):
        out[key] = res[key][b:b + 1, g * G:(g + 1) * G].double().numpy()
    out["lse"] = res["lse"][b:b + 1, g * G:(g + 1) * G].double().numpy()
    for key in ("dk", "dv"):
        out[key] = res[key][b:b + 1, g:g + 1].double().numpy()
    return out


def compare(case, got: dict, ref: dict, what: str = "") -> dict:
    errs = {k: rel_err(got[k], ref[k]) for k in ("o", "dq", "dk", "dv") if k in ref}
    if "lse" in ref:
        errs["lse"] = lse_err(got["lse"], ref["lse"])
    log(f"  {case.name} {what}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    return errs


def assert_within(case, errs: dict) -> None:
    tol = TOL[case.dtype]
    for k, v in errs.items():
        bound = LSE_TOL if k == "lse" else tol
        assert v <= bound, f"{case.name}: {k} error {v:.3e} > {bound:.1e}"


def dkdv_rows_by_head(case, x: dict, b: int, g: int, kv_rows, **extras):
    """orc.dkdv_rows for key rows of one (batch, kv head), as the sum of each query
    head's own contribution, the G heads computed in parallel threads (NumPy
    releases the interpreter lock inside its array loops and BLAS calls).
    ``extras``: bias, dropout_p and seed, as orc.dkdv_rows takes them."""
    from concurrent.futures import ThreadPoolExecutor
    G = case.Hq // case.Hkv

    def one(h):
        return orc.dkdv_rows(x["q"], x["k"], x["v"], x["do"], case.scale, case.causal, b, g,
                             kv_rows, heads=[h], **extras)

    with ThreadPoolExecutor(max_workers=G) as ex:
        parts = list(ex.map(one, range(g * G, (g + 1) * G)))
    return sum(p[0] for p in parts), sum(p[1] for p in parts)
