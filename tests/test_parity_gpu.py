"""HIP path against the fp64 oracle on the same seeded inputs, through the C ABI.

Gate: max|g - ref| / max|ref| <= 1e-2 (fp16) / 2e-2 (bf16) for O, dQ, dK, dV and
max|LSE - ref| <= 1e-3, on every workload family.  Shapes the oracle can afford
whole are compared element by element on sampled (batch, kv-head) groups; the
longest sequences are compared on sampled rows (O, LSE and dQ rows, and the
trailing key rows of dK/dV whose contributing queries are few under the causal
mask) plus identities that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle.attention_fp64 as orc
from exact_attention_backward_fa_amd import inputs
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

MODES = ("atomic", "separate")


def _run_groups(case, groups, device, modes=MODES):
    x = inputs.make_inputs(case)
    refs = {}
    for (b, g) in groups:
        pu.log(f"[oracle] {case.name} b={b} g={g}")
        refs[(b, g)] = pu.oracle_group(case, x, b, g)
    for mode in modes:
        pu.log(f"[gpu] {case.name} mode={mode} seed={case.seed}")
        res = pu.gpu_forward_backward(case, x, device, dq_mode=mode)
        for (b, g) in groups:
            errs = pu.compare(case, pu.gpu_group(case, res, b, g), refs[(b, g)],
                              f"{mode} b={b} g={g}")
            pu.assert_within(case, errs)


def test_single_head_oracle_fed(device):
    """One head, N=128, d=64, fp16: the backward is fed O and LSE from the oracle's
    forward (rounded to fp16 / fp32); the GPU forward is checked separately."""
    case = inputs.case_by_name("single")
    x = inputs.make_inputs(case)
    o_ref, lse_ref = orc.forward(x["q"], x["k"], x["v"], case.scale, case.causal)
    dq, dk, dv = orc.backward(x["q"], x["k"], x["v"], x["do"], case.scale, case.causal)
    ref = {"o": o_ref, "lse": lse_ref, "dq": dq, "dk": dk, "dv": dv}
    o_lse = (torch.from_numpy(o_ref).to(case.torch_dtype), torch.from_numpy(lse_ref).float())
    for mode in MODES:
        res = pu.gpu_forward_backward(case, x, device, dq_mode=mode, o_lse=o_lse)
        got = {k: res[k].double().numpy() for k in res}
        pu.assert_within(case, pu.compare(case, got, ref, f"oracle-fed {mode}"))
        res = pu.gpu_forward_backward(case, x, device, dq_mode=mode)
        got = {k: res[k].double().numpy() for k in res}
        pu.assert_within(case, pu.compare(case, got, ref, f"end-to-end {mode}"))


@pytest.mark.parametrize("name", [c.name for c in inputs.cases_of_family(2)])
def test_ragged(name, device):
    case = inputs.case_by_name(name)
    groups = [(b, g) for b in range(case.B) for g in range(case.Hkv)]
    _run_groups(case, groups, device)


def test_uniform_sequence_parallel_shape(device):
    case = inputs.case_by_name("uniform")
    _run_groups(case, [(0, 0), (1, 15)], device)


def _llama_groups(n):
    if n <= 1024:
        return [(0, 0), (3, 7), (2, 5)]
    if n <= 4096:
        return [(0, 0), (3, 7)]
    return [(1, 3)]


LLAMA_FULL = [c.name for c in inputs.cases_of_family(4) if c.Nq <= 8192]


@pytest.mark.parametrize("name", LLAMA_FULL)
def test_llama_gqa(name, device):
    case = inputs.case_by_name(name)
    _run_groups(case, _llama_groups(case.Nq), device)


def test_long_d64(device):
    case = inputs.case_by_name("long_d64_8192")
    _run_groups(case, [(0, 0), (0, 11)], device)


def _sampled_check(case, device, seed_rows=1234):
    """Row-sampled parity for sequences too long to materialise whole."""
    x = inputs.make_inputs(case)
    rng = np.random.default_rng(seed_rows + case.seed)
    N = case.Nq
    rows = np.unique(np.concatenate([[0, 1, N // 2, N - 2, N - 1], rng.integers(0, N, 27)]))
    tail = np.arange(N - 48, N)
    picks = [(0, 0, 0), (case.B - 1, case.Hq - 1, case.Hkv - 1)]
    ref = {}
    for (b, h, g) in picks:
        pu.log(f"[oracle] {case.name} rows b={b} h={h} g={g}")
        o, l_ = orc.forward_rows(x["q"], x["k"], x["v"], case.scale, case.causal, b, h, rows)
        dq = orc.dq_rows(x["q"], x["k"], x["v"], x["do"], case.scale, case.causal, b, h, rows)
        dk, dv = orc.dkdv_rows(x["q"], x["k"], x["v"], x["do"], case.scale, case.causal, b, g, tail)
        ref[(b, h, g)] = {"o": o, "lse": l_, "dq": dq, "dk": dk, "dv": dv}
    for mode in MODES:
        pu.log(f"[gpu] {case.name} mode={mode} seed={case.seed}")
        res = pu.gpu_forward_backward(case, x, device, dq_mode=mode)
        for (b, h, g), r in ref.items():
            got = {
                "o": res["o"][b, h, rows].double().numpy(),
                "lse": res["lse"][b, h, rows].double().numpy(),
                "dq": res["dq"][b, h, rows].double().numpy(),
                "dk": res["dk"][b, g, tail].double().numpy(),
                "dv": res["dv"][b, g, tail].double().numpy(),
            }
            pu.assert_within(case, pu.compare(case, got, r, f"{mode} rows b={b} h={h}"))
        _identities_any_size(case, x, res)


def _identities_any_size(case, x, res):
    """Per kv head: sum_j dK_j = 0 and <Q,dQ> = <K,dK>, <dO,O> = <V,dV> (no empty
    rows in these workloads).  Bounds allow for dtype rounding of the results."""
    G = case.Hq // case.Hkv
    tol = pu.TOL[case.dtype]
    for b in range(case.B):
        for g in range(case.Hkv):
            hs = slice(g * G, (g + 1) * G)
            dk = res["dk"][b, g].double()
            k = x["k"][b, g].double()
            scale_dk = dk.abs().sum(0).max().item()
            assert dk.sum(0).abs().max().item() <= tol * max(scale_dk, 1e-30)
            lhs = (x["q"][b, hs].double() * res["dq"][b, hs].double()).sum().item()
            rhs = (k * dk).sum().item()
            mag = (x["q"][b, hs].double() * res["dq"][b, hs].double()).abs().sum().item()
            assert abs(lhs - rhs) <= tol * max(mag, 1e-30)
            lhs = (x["do"][b, hs].double() * res["o"][b, hs].double()).sum().item()
            rhs = (x["v"][b, g].double() * res["dv"][b, g].double()).sum().item()
            mag = (x["do"][b, hs].double() * res["o"][b, hs].double()).abs().sum().item()
            assert abs(lhs - rhs) <= tol * max(mag, 1e-30)


@pytest.mark.parametrize("name", ["llama_gqa_fp16_16384", "llama_gqa_bf16_16384",
                                  "long_gqa_32768"])
def test_long_sampled(name, device):
    _sampled_check(inputs.case_by_name(name), device)


# --- edge cases --------------------------------------------------------------------

EDGE = [
    # B, Hq, Hkv, Nq, Nkv, d, dtype, causal
    (1, 4, 1, 1, 1, 64, "fp16", True),
    (1, 4, 1, 1, 1, 128, "bf16", False),
    (2, 4, 2, 5, 3, 64, "fp16", True),        # N_q > N_kv: two rows see no key
    (1, 2, 2, 300, 70, 128, "bf16", True),    # most rows see every key, top rows none
    (1, 8, 2, 129, 257, 128, "fp16", True),   # one past a tile on both sides
    (1, 8, 2, 127, 127, 128, "bf16", False),
    (3, 6, 3, 65, 200, 64, "bf16", True),
    (1, 2, 1, 513, 31, 64, "fp16", False),
    (1, 4, 4, 64, 128, 128, "fp16", True),
    # around the 256-row key blocks of the dK/dV kernel and query blocks of the dQ pass
    (1, 4, 1, 257, 513, 128, "bf16", True),
    (2, 8, 2, 255, 255, 64, "fp16", True),
    (1, 2, 1, 1000, 300, 128, "fp16", True),  # N_q > N_kv: the first 700 rows see no key
    (1, 2, 2, 64, 700, 128, "bf16", False),
    (1, 8, 8, 320, 320, 128, "bf16", True),
]


@pytest.mark.parametrize("shape", EDGE, ids=[f"{s[0]}x{s[1]}x{s[2]}_{s[3]}x{s[4]}_d{s[5]}_{s[6]}_{'c' if s[7] else 'nc'}" for s in EDGE])
def test_edge_shapes(shape, device):
    B, Hq, Hkv, Nq, Nkv, d, dt, causal = shape
    x = inputs.make_custom(77 + Nq + Nkv, B, Hq, Hkv, Nq, Nkv, d, dt)
    case = inputs.Case("edge", 0, 0, B, Hq, Hkv, Nq, Nkv, d, dt, causal, 1.0 / np.sqrt(d))
    o, lse = orc.forward(x["q"], x["k"], x["v"], case.scale, causal)
    dq, dk, dv = orc.backward(x["q"], x["k"], x["v"], x["do"], case.scale, causal)
    ref = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    for mode in MODES:
        res = pu.gpu_forward_backward(case, x, device, dq_mode=mode)
        got = {k: res[k].double().numpy() for k in res}
        pu.assert_within(case, pu.compare(case, got, ref, mode))


@pytest.mark.parametrize("causal", [False, True])
def test_rising_logits(causal, device):
    """Scores that rise by about 115 log2 units along every row: the forward's
    per-column softmax reference, set from the first pair of keys, is then exceeded
    by more than its 64-unit headroom and the workgroup reruns its item with raised
    references.  Forward and backward must still match the oracle."""
    B, Hq, Hkv, N, d = 1, 2, 1, 384, 64
    g = torch.Generator().manual_seed(4242)
    u = torch.full((d,), 1.0 / np.sqrt(d))
    ramp = torch.arange(N, dtype=torch.float32) / N
    x = {
        "q": (5.0 * u + 0.5 * torch.randn(B, Hq, N, d, generator=g)).to(torch.bfloat16),
        "k": (16.0 * ramp[:, None] * u + 0.5 * torch.randn(B, Hkv, N, d, generator=g)).to(torch.bfloat16),
        "v": torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16),
        "do": torch.randn(B, Hq, N, d, generator=g).to(torch.bfloat16),
    }
    case = inputs.Case("rising", 0, 0, B, Hq, Hkv, N, N, d, "bf16", causal, 1.0)
    o, lse = orc.forward(x["q"], x["k"], x["v"], case.scale, causal)
    dq, dk, dv = orc.backward(x["q"], x["k"], x["v"], x["do"], case.scale, causal)
    ref = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    res = pu.gpu_forward_backward(case, x, device)
    got = {k: res[k].double().numpy() for k in res}
    pu.assert_within(case, pu.compare(case, got, ref))


@pytest.mark.parametrize("dims", [(0, 4, 2, 16, 16), (2, 4, 2, 0, 16), (2, 4, 2, 16, 0),
                                  (2, 4, 2, 0, 0)])
def test_zero_sizes(dims, device):
    import exact_attention_backward_fa_amd as fa
    B, Hq, Hkv, Nq, Nkv = dims
    d = 64
    q = torch.randn(B, Hq, Nq, d, device=device).half()
    k = torch.randn(B, Hkv, Nkv, d, device=device).half()
    v = torch.randn(B, Hkv, Nkv, d, device=device).half()
    do = torch.randn(B, Hq, Nq, d, device=device).half()
    for causal in (False, True):
        o, lse = fa.fwd(q, k, v, 0.125, causal)
        for mode in MODES:
            dq = torch.full_like(q, float("nan"))
            dk = torch.full_like(k, float("nan"))
            dv = torch.full_like(v, float("nan"))
            fa.bwd_into(q, k, v, o, lse, do, dq, dk, dv, 0.125, causal, dq_mode=mode)
            torch.cuda.synchronize()
            assert bool((dk == 0).all()) and bool((dv == 0).all())
            assert bool((dq == 0).all())
        if Nkv == 0:
            assert bool((o == 0).all()) and bool((lse == float("-inf")).all())


def _guarded(shape, dtype, device, pad=64, fill=12345.0):
    n = int(np.prod(shape))
    buf = torch.full((pad + n + pad,), fill, dtype=dtype, device=device)
    return buf, buf[pad:pad + n].view(shape)


@pytest.mark.parametrize("mode", MODES)
def test_no_writes_outside_outputs(mode, device):
    """Ragged tails must not write past the end of any output (canary bands)."""
    import exact_attention_backward_fa_amd as fa
    B, Hq, Hkv, Nq, Nkv, d = 1, 4, 2, 100, 333, 64
    x = pu.to_dev(inputs.make_custom(5, B, Hq, Hkv, Nq, Nkv, d, "fp16"), device)
    for causal in (True, False):
        ob, o = _guarded((B, Hq, Nq, d), torch.float16, device)
        lb, lse = _guarded((B, Hq, Nq), torch.float32, device)
        fa.fwd_into(x["q"], x["k"], x["v"], o, lse, 0.125, causal)
        dqb, dq = _guarded((B, Hq, Nq, d), torch.float16, device)
        dkb, dk = _guarded((B, Hkv, Nkv, d), torch.float16, device)
        dvb, dv = _guarded((B, Hkv, Nkv, d), torch.float16, device)
        fa.bwd_into(x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, 0.125, causal, dq_mode=mode)
        torch.cuda.synchronize()
        for buf in (ob, lb, dqb, dkb, dvb):
            assert bool((buf[:64] == 12345.0).all()) and bool((buf[-64:] == 12345.0).all())


def test_separate_path_is_bitwise_repeatable(device):
    import exact_attention_backward_fa_amd as fa
    case = inputs.case_by_name("llama_gqa_bf16_1024")
    x = pu.to_dev(inputs.make_inputs(case), device)
    o, lse = fa.fwd(x["q"], x["k"], x["v"], case.scale, True)
    a = fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], case.scale, True, dq_mode="separate")
    b = fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], case.scale, True, dq_mode="separate")
    c = fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], case.scale, True, dq_mode="atomic")
    d = fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], case.scale, True, dq_mode="atomic")
    for t1, t2 in zip(a, b):
        assert torch.equal(t1.view(torch.int16), t2.view(torch.int16))
    # dK and dV never use atomics, so they repeat bitwise on the atomic path too
    for t1, t2 in zip(c[1:], d[1:]):
        assert torch.equal(t1.view(torch.int16), t2.view(torch.int16))
    # the two paths compute dK/dV with different kernels (different summation
    # order): they agree to rounding
    for t1, t2 in zip(a, c):
        err = float((t1.float() - t2.float()).abs().max() / t2.float().abs().max())
        assert err <= 1e-2, err


def test_outputs_need_no_initialisation(device):
    import exact_attention_backward_fa_amd as fa
    case = inputs.case_by_name("ragged_100x333_c")
    x = pu.to_dev(inputs.make_inputs(case), device)
    o, lse = fa.fwd(x["q"], x["k"], x["v"], case.scale, True)
    clean = fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], case.scale, True, dq_mode="atomic")
    for mode in MODES:
        outs = [torch.full_like(t, float("nan")) for t in clean]
        ws = torch.full((fa.bwd_workspace_bytes(case.B, case.Hq, case.Hkv, case.Nq, case.Nkv, case.d,
                                                True, case.torch_dtype, mode),), 0xFF,
                        dtype=torch.uint8, device=device)
        fa.bwd_into(x["q"], x["k"], x["v"], o, lse, x["do"], *outs, case.scale, True,
                    dq_mode=mode, workspace=ws)
        torch.cuda.synchronize()
        for t, ref in zip(outs, clean):
            assert bool(torch.isfinite(t).all())
            assert (t.float() - ref.float()).abs().max().item() <= 1e-2 * ref.float().abs().max().item()


def test_rejected_call_writes_nothing(device):
    import exact_attention_backward_fa_amd as fa
    from exact_attention_backward_fa_amd import _lib
    case = inputs.case_by_name("ragged_17x17_c")
    x = pu.to_dev(inputs.make_inputs(case), device)
    o, lse = fa.fwd(x["q"], x["k"], x["v"], case.scale, True)
    dq = torch.full_like(x["q"], 7.0)
    dk = torch.full_like(x["k"], 7.0)
    dv = torch.full_like(x["v"], 7.0)
    ws = torch.empty(16, dtype=torch.uint8, device=device)  # far too small
    with pytest.raises(RuntimeError, match="status -6"):
        fa.bwd_into(x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, case.scale, True,
                    dq_mode="atomic", workspace=ws)
    torch.cuda.synchronize()
    assert bool((dq == 7).all()) and bool((dk == 7).all()) and bool((dv == 7).all())
    assert _lib.status_string(-6).startswith("workspace")
