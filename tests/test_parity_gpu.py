"""HIP path against the fp64 oracle on the same seeded inputs, through the C ABI.

Gate: max|g - ref| / max|ref| <= 1e-2 (fp16) / 2e-2 (bf16) for O, dQ, dK, dV and
max|LSE - ref| <= 1e-3, on every workload family.  Shapes the oracle can afford
whole are compared element by element on sampled (batch, kv-head) groups; the
longest sequences are compared on sampled rows (O, LSE and dQ rows; the
leading key rows of dK/dV, which accumulate over every query tile of the group,
and the trailing ones, which see the fewest) plus identities that hold at any
size.
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


def _sampled_check(case, device, lead, seed_rows=1234):
    """Row-sampled parity for sequences too long to materialise whole.

    Key rows compared element by element: the trailing 48 (the fewest
    contributing queries under the causal mask) and, for the first sampled group,
    the leading ``lead`` (every query of the group's G heads contributes: the
    dK/dV kernel's longest accumulations)."""
    x = inputs.make_inputs(case)
    rng = np.random.default_rng(seed_rows + case.seed)
    N = case.Nq
    rows = np.unique(np.concatenate([[0, 1, N // 2, N - 2, N - 1], rng.integers(0, N, 27)]))
    tail = np.arange(N - 48, N)
    picks = [(0, 0, 0), (case.B - 1, case.Hq - 1, case.Hkv - 1)]
    ref = {}
    keys = {}
    for n, (b, h, g) in enumerate(picks):
        kv_rows = np.concatenate([np.arange(lead), tail]) if n == 0 else tail
        keys[(b, h, g)] = kv_rows
        pu.log(f"[oracle] {case.name} rows b={b} h={h} g={g} ({len(kv_rows)} key rows)")
        o, l_ = orc.forward_rows(x["q"], x["k"], x["v"], case.scale, case.causal, b, h, rows)
        dq = orc.dq_rows(x["q"], x["k"], x["v"], x["do"], case.scale, case.causal, b, h, rows)
        dk, dv = pu.dkdv_rows_by_head(case, x, b, g, kv_rows)
        ref[(b, h, g)] = {"o": o, "lse": l_, "dq": dq, "dk": dk, "dv": dv}
    for mode in MODES:
        pu.log(f"[gpu] {case.name} mode={mode} seed={case.seed}")
        res = pu.gpu_forward_backward(case, x, device, dq_mode=mode)
        for (b, h, g), r in ref.items():
            kv_rows = keys[(b, h, g)]
            got = {
                "o": res["o"][b, h, rows].double().numpy(),
                "lse": res["lse"][b, h, rows].double().numpy(),
                "dq": res["dq"][b, h, rows].double().numpy(),
                "dk": res["dk"][b, g, kv_rows].double().numpy(),
                "dv": res["dv"][b, g, kv_rows].double().numpy(),
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


@pytest.mark.parametrize("name,lead", [("llama_gqa_fp16_16384", 64), ("llama_gqa_bf16_16384", 64),
                                       ("long_gqa_32768", 16)])
def test_long_sampled(name, lead, device):
    _sampled_check(inputs.case_by_name(name), device, lead)


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


# Head dims beyond 64 and 128 (the Liger-Kernel pull request "[Kernel] Flash
# attention 2", Details, claims no restriction on the head dimension).  d = 32 and
# 96 run the same kernels with one and three 32-wide contraction steps; d = 160,
# 192, 224 and 256 keep 32 resident rows per wave and double-buffered tiles.
# Shapes are ragged on both sides and span several 256-row (d > 128: 128-row) work
# items.
HEAD_DIM_CASES = [
    # B, Hq, Hkv, Nq, Nkv, d, dtype, causal
    (2, 4, 2, 100, 333, 32, "fp16", True),
    (1, 8, 2, 700, 700, 32, "bf16", False),
    (2, 4, 1, 513, 257, 32, "bf16", True),     # N_q > N_kv: the first rows see no key
    (2, 4, 2, 100, 333, 96, "bf16", True),
    (1, 6, 3, 700, 700, 96, "fp16", False),
    (1, 4, 4, 300, 1000, 96, "fp16", True),
    (2, 4, 2, 100, 333, 256, "fp16", True),
    (1, 4, 2, 600, 600, 256, "bf16", True),
    (1, 2, 1, 333, 450, 256, "bf16", False),
    (1, 4, 4, 129, 64, 256, "fp16", True),      # N_q > N_kv
    (2, 4, 2, 100, 333, 160, "bf16", True),
    (1, 4, 2, 300, 300, 160, "fp16", False),
    (1, 4, 1, 400, 700, 192, "fp16", True),
    (1, 2, 2, 257, 129, 192, "bf16", True),     # N_q > N_kv
    (2, 4, 2, 300, 300, 224, "bf16", False),
    (1, 4, 4, 100, 333, 224, "fp16", True),
]


@pytest.mark.parametrize("shape", HEAD_DIM_CASES,
                         ids=[f"d{s[5]}_{s[0]}x{s[1]}x{s[2]}_{s[3]}x{s[4]}_{s[6]}_{'c' if s[7] else 'nc'}"
                              for s in HEAD_DIM_CASES])
def test_head_dims(shape, device):
    B, Hq, Hkv, Nq, Nkv, d, dt, causal = shape
    x = inputs.make_custom(991 + d + Nq, B, Hq, Hkv, Nq, Nkv, d, dt)
    case = inputs.Case(f"d{d}", 0, 0, B, Hq, Hkv, Nq, Nkv, d, dt, causal, 1.0 / np.sqrt(d))
    o, lse = orc.forward(x["q"], x["k"], x["v"], case.scale, causal)
    dq, dk, dv = orc.backward(x["q"], x["k"], x["v"], x["do"], case.scale, causal)
    ref = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    modes = MODES if d in (64, 128) else ("separate", "auto")
    for mode in modes:
        res = pu.gpu_forward_backward(case, x, device, dq_mode=mode)
        got = {k: res[k].double().numpy() for k in res}
        pu.assert_within(case, pu.compare(case, got, ref, mode))


def test_head_dim_256_long_sequence(device):
    """d = 256 at N = 4096, causal GQA bf16: many work items per head, double
    buffering over 64 key tiles; one group compared in full."""
    B, Hq, Hkv, N, d = 1, 8, 2, 4096, 256
    x = inputs.make_custom(256_4096, B, Hq, Hkv, N, N, d, "bf16")
    case = inputs.Case("d256_4096", 0, 0, B, Hq, Hkv, N, N, d, "bf16", True, 1.0 / np.sqrt(d))
    ref = pu.oracle_group(case, x, 0, 1)
    res = pu.gpu_forward_backward(case, x, device, dq_mode="separate")
    pu.assert_within(case, pu.compare(case, pu.gpu_group(case, res, 0, 1), ref, "separate g=1"))


def test_atomic_path_only_for_d64_d128(device):
    import exact_attention_backward_fa_amd as fa
    x = pu.to_dev(inputs.make_custom(5, 1, 2, 1, 64, 64, 96, "fp16"), device)
    o, lse = fa.fwd(x["q"], x["k"], x["v"], 0.1, True)
    with pytest.raises(RuntimeError, match="status -3"):
        fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], 0.1, True, dq_mode="atomic")


RISING = [("bf16", 80.0), ("fp16", 12.0), ("fp16", 30.0)]


@pytest.mark.parametrize("dtype,rise", RISING, ids=[f"{d}_{r:g}nats" for d, r in RISING])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_logits(dtype, rise, causal, device):
    """Scores that rise by about ``rise`` nats along every row.  The forward sets
    each query column's softmax reference from the first pair of keys it sees and
    lets a later score exceed it by a type-dependent headroom (64 log2 units for
    bf16, 15 for fp16, whose P would be infinite from 2^16 on); a larger rise
    makes the workgroup rerun its item with raised references.  12 nats (17.3 log2
    units) passes the fp16 headroom, 30 and 80 pass it by far, and 80 nats passes
    the bf16 one.  Forward and backward must still match the oracle on both dQ
    paths."""
    B, Hq, Hkv, N, d = 1, 2, 1, 384, 64
    g = torch.Generator().manual_seed(4242)
    u = torch.full((d,), 1.0 / np.sqrt(d))
    ramp = torch.arange(N, dtype=torch.float32) / N
    # score ~ (5 u) . (amp * ramp * u) = 5 * amp * ramp nats, plus noise
    amp = rise / 5.0
    tdt = inputs.TORCH_DTYPE[dtype]
    x = {
        "q": (5.0 * u + 0.5 * torch.randn(B, Hq, N, d, generator=g)).to(tdt),
        "k": (amp * ramp[:, None] * u + 0.5 * torch.randn(B, Hkv, N, d, generator=g)).to(tdt),
        "v": torch.randn(B, Hkv, N, d, generator=g).to(tdt),
        "do": torch.randn(B, Hq, N, d, generator=g).to(tdt),
    }
    case = inputs.Case("rising", 0, 0, B, Hq, Hkv, N, N, d, dtype, causal, 1.0)
    o, lse = orc.forward(x["q"], x["k"], x["v"], case.scale, causal)
    dq, dk, dv = orc.backward(x["q"], x["k"], x["v"], x["do"], case.scale, causal)
    ref = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    # most rows really pass the headroom: a later score exceeds the maximum over
    # the first 32 keys by more than H log2 units (H = 15 fp16, 64 bf16)
    sc = orc.as_f64(x["q"][0]) @ orc.as_f64(x["k"][0, 0]).T
    over = (sc[:, :, 32:].max(-1) - sc[:, :, :32].max(-1)) / np.log(2.0)
    assert (over > (15.0 if dtype == "fp16" else 64.0)).mean() > 0.5
    for mode in MODES:
        res = pu.gpu_forward_backward(case, x, device, dq_mode=mode)
        got = {k: res[k].double().numpy() for k in res}
        assert all(bool(np.isfinite(got[k]).all()) for k in ("o", "dq", "dk", "dv"))
        pu.assert_within(case, pu.compare(case, got, ref, mode))


@pytest.mark.parametrize("causal", [False, True])
def test_row_sum_check_without_overflow(causal, device):
    """fp16 scores that rise about 8 nats (11.5 log2 units) along every row: below
    the fp16 headroom of 15, so no P can overflow, yet the row sums pass 2^15.
    The plain forward's fast first pass checks the row sums, so it marks these
    items and the second launch recomputes them with the per-pair test; O, LSE and
    the gradients must match the oracle on both dQ paths."""
    B, Hq, Hkv, N, d = 1, 2, 1, 384, 64
    g = torch.Generator().manual_seed(4343)
    u = torch.full((d,), 1.0 / np.sqrt(d))
    ramp = torch.arange(N, dtype=torch.float32) / N
    amp = 8.0 / 5.0
    x = {
        "q": (5.0 * u + 0.1 * torch.randn(B, Hq, N, d, generator=g)).half(),
        "k": (amp * ramp[:, None] * u + 0.1 * torch.randn(B, Hkv, N, d, generator=g)).half(),
        "v": torch.randn(B, Hkv, N, d, generator=g).half(),
        "do": torch.randn(B, Hq, N, d, generator=g).half(),
    }
    case = inputs.Case("sum_check", 0, 0, B, Hq, Hkv, N, N, d, "fp16", causal, 1.0)
    o, lse = orc.forward(x["q"], x["k"], x["v"], case.scale, causal)
    dq, dk, dv = orc.backward(x["q"], x["k"], x["v"], x["do"], case.scale, causal)
    ref = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    # the premise, non-causal rows over all keys: no later score exceeds the first
    # 32 keys' maximum by 15 log2 units, yet the sum of 2^(score - that maximum)
    # over the row passes 2^15
    sc = orc.as_f64(x["q"][0]) @ orc.as_f64(x["k"][0, 0]).T / np.log(2.0)
    ref_max = sc[:, :, :32].max(-1, keepdims=True)
    assert (sc.max(-1, keepdims=True) - ref_max).max() < 15.0
    assert (np.exp2(sc - ref_max).sum(-1) > 2.0 ** 15).mean() > 0.5
    for mode in MODES:
        res = pu.gpu_forward_backward(case, x, device, dq_mode=mode)
        got = {k: res[k].double().numpy() for k in res}
        assert all(bool(np.isfinite(got[k]).all()) for k in ("o", "dq", "dk", "dv"))
        pu.assert_within(case, pu.compare(case, got, ref, mode))


def test_fa_bwd_entry_point(device):
    """fa_bwd itself (the dQ path FA_DQ_AUTO picks, workspace of exactly
    fa_bwd_workspace_bytes bytes), called through ctypes, against the oracle."""
    import ctypes

    import exact_attention_backward_fa_amd as fa
    from exact_attention_backward_fa_amd import _lib
    lib = _lib.load()
    for name, groups in (("ragged_100x333_c", [(0, 1), (1, 3)]), ("llama_gqa_bf16_1024", [(2, 5)])):
        case = inputs.case_by_name(name)
        x = inputs.make_inputs(case)
        d = pu.to_dev(x, device)
        o, lse = fa.fwd(d["q"], d["k"], d["v"], case.scale, case.causal)
        dq = torch.full_like(d["q"], float("nan"))
        dk = torch.full_like(d["k"], float("nan"))
        dv = torch.full_like(d["v"], float("nan"))
        dt = _lib.FA_DTYPE[case.torch_dtype]
        need = lib.fa_bwd_workspace_bytes(case.B, case.Hq, case.Hkv, case.Nq, case.Nkv, case.d,
                                          int(case.causal), dt)
        assert need > 0
        ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=device)
        stream = torch.cuda.current_stream(device).cuda_stream
        rc = lib.fa_bwd(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), o.data_ptr(),
                        lse.data_ptr(), d["do"].data_ptr(), dq.data_ptr(), dk.data_ptr(),
                        dv.data_ptr(), case.B, case.Hq, case.Hkv, case.Nq, case.Nkv, case.d,
                        ctypes.c_float(case.scale), int(case.causal), dt, ws.data_ptr(),
                        ctypes.c_size_t(need), stream)
        assert rc == 0, _lib.status_string(rc)
        # one byte short of the requirement is rejected before any launch
        rc = lib.fa_bwd(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), o.data_ptr(),
                        lse.data_ptr(), d["do"].data_ptr(), dq.data_ptr(), dk.data_ptr(),
                        dv.data_ptr(), case.B, case.Hq, case.Hkv, case.Nq, case.Nkv, case.d,
                        ctypes.c_float(case.scale), int(case.causal), dt, ws.data_ptr(),
                        ctypes.c_size_t(need - 1), stream)
        assert rc == -6
        torch.cuda.synchronize(device)
        res = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
        for (b, g) in groups:
            ref = pu.oracle_group(case, x, b, g)
            pu.assert_within(case, pu.compare(case, pu.gpu_group(case, res, b, g), ref,
                                              f"fa_bwd b={b} g={g}"))


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
