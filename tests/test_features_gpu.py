"""Additive score bias (with its gradient dBias = dS) and dropout of P on the GPU
against the fp64 oracle, through the C ABI (fa_fwd_bias_dropout /
fa_bwd_bias_dropout) and the autograd wrapper.

The Liger-Kernel pull request "[Kernel] Flash attention 2", Details, lists an
attention mask / bias and dropout; the oracle's readings (bias added to the scaled
scores; dropout of P after the softmax with the Philox4x32-10 keep rule) are pinned
in tests/oracle_pins.py.  The keep decisions must agree bit for bit, or the outputs
would differ by whole dropped terms, far outside the bounds.  Bounds as for the
plain path: max|g - ref| / max|ref| <= 1e-2 (fp16), 2e-2 (bf16); LSE 1e-3 absolute.
"""
import numpy as np
import pytest
import torch

import oracle.attention_fp64 as orc
from exact_attention_backward_fa_amd import inputs
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


def _bias(seed, shape, Nkv, dtype, mult=2.0, pad_keys=None):
    """A bias of `shape` (its last dimension N_kv) in the given dtype, stored with
    rows padded to a multiple of 8 elements (16-byte rows).  ``pad_keys``: keys set
    to -inf (a key-padding mask) in every row."""
    g = torch.Generator().manual_seed(seed)
    pad = (Nkv + 7) // 8 * 8
    store = (mult * torch.randn(*shape[:-1], pad, generator=g)).to(inputs.TORCH_DTYPE[dtype])
    b = store[..., :Nkv]
    if pad_keys is not None:
        b[..., pad_keys] = float("-inf")
    return b


def _bias_to(bias, device):
    """The bias view on the device over a copy of its whole padded storage."""
    store = bias._base if bias._base is not None else bias
    return store.to(device)[..., :bias.shape[-1]]


def _run(case, x, bias, dropout_p, seed, device, want_dbias):
    import exact_attention_backward_fa_amd as fa
    d = pu.to_dev(x, device)
    bd = None if bias is None else _bias_to(bias, device)
    o, lse = fa.fwd_bias_dropout(d["q"], d["k"], d["v"], case.scale, case.causal, bias=bd,
                                 dropout_p=dropout_p, seed=seed)
    dq, dk, dv, dbias = fa.bwd_bias_dropout(d["q"], d["k"], d["v"], o, lse, d["do"], case.scale,
                                            case.causal, bias=bd, want_dbias=want_dbias,
                                            dropout_p=dropout_p, seed=seed)
    torch.cuda.synchronize(device)
    out = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    if dbias is not None:
        out["dbias"] = dbias.cpu()
    return out


def _oracle(case, x, bias, dropout_p, seed, want_dbias):
    b = None if bias is None else orc.as_f64(bias)
    o, lse = orc.forward(x["q"], x["k"], x["v"], case.scale, case.causal, bias=b,
                         dropout_p=dropout_p, seed=seed)
    res = orc.backward(x["q"], x["k"], x["v"], x["do"], case.scale, case.causal, bias=b,
                       dropout_p=dropout_p, seed=seed, return_dbias=want_dbias)
    ref = {"o": o, "lse": lse, "dq": res[0], "dk": res[1], "dv": res[2]}
    if want_dbias:
        ref["dbias"] = res[3]
    return ref


def _compare(case, got, ref, what):
    g = {k: v.double().numpy() for k, v in got.items()}
    errs = pu.compare(case, g, ref, what)
    if "dbias" in ref:
        errs["dbias"] = pu.rel_err(g["dbias"], ref["dbias"])
        pu.log(f"    dbias={errs['dbias']:.2e}")
    pu.assert_within(case, errs)
    return g


BIAS_CASES = [
    # name, B, Hq, Hkv, Nq, Nkv, d, dtype, causal, bias shape (None: full), dropout p
    ("full_gqa_c", 2, 4, 2, 100, 333, 64, "fp16", True, None, 0.0),
    ("full_nc", 1, 4, 4, 300, 257, 128, "bf16", False, None, 0.0),
    ("shared_heads_c", 2, 4, 1, 257, 513, 128, "fp16", True, "1h", 0.0),
    ("key_padding", 2, 4, 2, 200, 333, 64, "bf16", False, "keys", 0.0),
    ("row_bias_c", 1, 8, 2, 129, 129, 128, "bf16", True, "rows", 0.0),
    ("dropout_c", 2, 4, 2, 100, 333, 64, "fp16", True, "none", 0.2),
    ("dropout_nc", 1, 4, 4, 257, 700, 128, "bf16", False, "none", 0.5),
    ("bias_dropout_c", 2, 4, 2, 300, 300, 128, "fp16", True, None, 0.1),
    ("bias_dropout_gqa", 1, 8, 2, 513, 257, 64, "bf16", True, "keys", 0.3),
    ("dropout_nq_gt_nkv", 1, 4, 1, 200, 64, 64, "fp16", True, "none", 0.25),
    # dBias without a bias (the bias instance with a null bias): dS of plain attention
    ("dbias_only_c", 1, 4, 2, 130, 200, 64, "bf16", True, "none", 0.0),
    # a bias rising along the keys by far more than the forward's headroom over the
    # first visible pair (fp16: 10.4 nats, bf16: 44 nats): the rerun path with a bias
    ("rising_bias_fp16", 1, 4, 2, 200, 333, 64, "fp16", False, "ramp", 0.0),
    ("rising_bias_bf16_c", 1, 4, 2, 300, 300, 128, "bf16", True, "ramp", 0.1),
    # dBias rows longer than one 8192-key block of the masked-entry fill, rows
    # alternating between two 16-byte alignments (8204 keys), 8-byte dBias stores
    ("long_rows_dbias_c", 1, 1, 1, 8204, 8204, 64, "fp16", True, None, 0.0),
]


def _bias_for(kind, B, Hq, Nq, Nkv, dt, seed):
    if kind == "none":
        return None
    if kind is None:
        return _bias(seed, (B, Hq, Nq, Nkv), Nkv, dt)
    if kind == "1h":
        return _bias(seed, (B, 1, Nq, Nkv), Nkv, dt)
    if kind == "keys":  # per-key bias with a padding mask on the last keys of a batch row
        return _bias(seed, (B, 1, 1, Nkv), Nkv, dt, pad_keys=[Nkv - 1, Nkv - 2, Nkv - 5, 3])
    if kind == "rows":
        return _bias(seed, (1, 1, Nq, Nkv), Nkv, dt)
    if kind == "ramp":  # 0.25 nats per key (83 nats over 333 keys) plus noise
        b = _bias(seed, (B, 1, Nq, Nkv), Nkv, dt, mult=0.5)
        b += (0.25 * torch.arange(Nkv, dtype=torch.float32)).to(b.dtype)
        return b
    raise ValueError(kind)


@pytest.mark.parametrize("cfg", BIAS_CASES, ids=[c[0] for c in BIAS_CASES])
def test_bias_dropout_parity(cfg, device):
    name, B, Hq, Hkv, Nq, Nkv, d, dt, causal, kind, p = cfg
    x = inputs.make_custom(7000 + Nq + Nkv + d, B, Hq, Hkv, Nq, Nkv, d, dt)
    case = inputs.Case(name, 0, 0, B, Hq, Hkv, Nq, Nkv, d, dt, causal, 1.0 / np.sqrt(d))
    bias = _bias_for(kind, B, Hq, Nq, Nkv, dt, 31 + Nq)
    seed = (0x9E3779B9 << 32) | (1234 + Nq)
    want = True
    ref = _oracle(case, x, bias, p, seed, want)
    got = _run(case, x, bias, p, seed, device, want)
    g = _compare(case, got, ref, name)
    if causal:  # keys the mask hides have a zero gradient
        i = np.arange(Nq)[:, None]
        j = np.arange(Nkv)[None, :]
        hidden = np.broadcast_to(j > i + (Nkv - Nq), g["dbias"].shape)
        assert np.all(g["dbias"][hidden] == 0)


# A bias per (batch, key) with no gradient wanted (a key-padding mask, say) runs on
# the key-bias instances, at every head dim: the plain kernels' shape, the bias read once per
# key tile (forward, dQ pass: it starts the score accumulator) or held per key
# (dK/dV kernel).
KEY_BIAS_CASES = [
    # name, B, Hq, Hkv, Nq, Nkv, d, dtype, causal, kind
    ("kb_gqa_c", 2, 4, 2, 200, 333, 64, "fp16", True, "keys"),
    ("kb_nc", 1, 4, 4, 300, 257, 128, "bf16", False, "keys"),
    ("kb_nq_gt_nkv_c", 1, 8, 2, 513, 257, 128, "bf16", True, "keys"),
    ("kb_d64_bf16_c", 2, 4, 1, 129, 700, 64, "bf16", True, "keys"),
    ("kb_long_c", 1, 8, 2, 2048, 2048, 128, "fp16", True, "keys"),
    # rising along the keys by 0.25 nats per key: the forward's rerun with a key bias
    ("kb_ramp_fp16", 1, 4, 2, 200, 333, 64, "fp16", False, "keyramp"),
    ("kb_ramp_bf16_c", 1, 4, 2, 300, 300, 128, "bf16", True, "keyramp"),
    # the other head dims (the key-bias instances exist at every d)
    ("kb_d32_c", 2, 4, 2, 200, 333, 32, "bf16", True, "keys"),
    ("kb_d96_nc", 1, 4, 4, 300, 257, 96, "fp16", False, "keys"),
    ("kb_d160_c", 1, 4, 2, 257, 300, 160, "fp16", True, "keys"),
    ("kb_d192_nc", 1, 4, 1, 300, 400, 192, "bf16", False, "keys"),
    ("kb_d224_c", 1, 2, 2, 129, 257, 224, "bf16", True, "keys"),
    ("kb_d256_c", 1, 4, 2, 300, 300, 256, "fp16", True, "keyramp"),
]


@pytest.mark.parametrize("cfg", KEY_BIAS_CASES, ids=[c[0] for c in KEY_BIAS_CASES])
def test_key_bias_parity(cfg, device):
    name, B, Hq, Hkv, Nq, Nkv, d, dt, causal, kind = cfg
    x = inputs.make_custom(9000 + Nq + Nkv + d, B, Hq, Hkv, Nq, Nkv, d, dt)
    case = inputs.Case(name, 0, 0, B, Hq, Hkv, Nq, Nkv, d, dt, causal, 1.0 / np.sqrt(d))
    if kind == "keys":
        bias = _bias_for("keys", B, Hq, Nq, Nkv, dt, 17 + Nq)
    else:
        bias = _bias(17 + Nq, (B, 1, 1, Nkv), Nkv, dt, mult=0.5)
        bias += (0.25 * torch.arange(Nkv, dtype=torch.float32)).to(bias.dtype)
    ref = _oracle(case, x, bias, 0.0, 0, False)
    got = _run(case, x, bias, 0.0, 0, device, False)
    _compare(case, got, ref, name)


# Dropout without a bias: the forward and the dQ pass keep the plain 64-row
# shape (the dK/dV kernel at d = 64 as well).
DROP_ONLY_CASES = [
    # name, B, Hq, Hkv, Nq, Nkv, d, dtype, causal, p
    ("drop_gqa_c", 2, 4, 2, 100, 333, 64, "fp16", True, 0.2),
    ("drop_nc", 1, 4, 4, 257, 700, 128, "bf16", False, 0.5),
    ("drop_nq_gt_nkv_c", 1, 4, 1, 200, 64, 64, "fp16", True, 0.25),
    ("drop_d64_bf16_c", 2, 4, 2, 300, 300, 64, "bf16", True, 0.3),
    ("drop_long_c", 1, 8, 2, 2048, 2048, 128, "bf16", True, 0.1),
]


@pytest.mark.parametrize("cfg", DROP_ONLY_CASES, ids=[c[0] for c in DROP_ONLY_CASES])
def test_dropout_only_parity(cfg, device):
    name, B, Hq, Hkv, Nq, Nkv, d, dt, causal, p = cfg
    x = inputs.make_custom(9500 + Nq + Nkv + d, B, Hq, Hkv, Nq, Nkv, d, dt)
    case = inputs.Case(name, 0, 0, B, Hq, Hkv, Nq, Nkv, d, dt, causal, 1.0 / np.sqrt(d))
    seed = (0x85EBCA6B << 32) | (77 + Nq)
    ref = _oracle(case, x, None, p, seed, False)
    got = _run(case, x, None, p, seed, device, False)
    _compare(case, got, ref, name)


def test_autograd_dropout_without_bias(device):
    """attention(..., dropout_p=, seed=) with no bias against the oracle."""
    from exact_attention_backward_fa_amd import attention
    B, Hq, Hkv, Nq, Nkv, d = 2, 4, 2, 190, 256, 128
    x = inputs.make_custom(79, B, Hq, Hkv, Nq, Nkv, d, "fp16")
    case = inputs.Case("autograd_dropout", 0, 0, B, Hq, Hkv, Nq, Nkv, d, "fp16", True, 1.0 / np.sqrt(d))
    ref = _oracle(case, x, None, 0.2, 31337, False)
    q, k, v = (x[n].to(device).requires_grad_() for n in ("q", "k", "v"))
    o = attention(q, k, v, causal=True, dropout_p=0.2, seed=31337)
    (o.float() * x["do"].to(device).float()).sum().backward()
    torch.cuda.synchronize(device)
    got = {"o": o.detach().double().cpu().numpy(), "dq": q.grad.double().cpu().numpy(),
           "dk": k.grad.double().cpu().numpy(), "dv": v.grad.double().cpu().numpy()}
    r = {kk: ref[kk] for kk in ("o", "dq", "dk", "dv")}
    pu.assert_within(case, pu.compare(case, got, r, "autograd dropout"))


def test_key_bias_fully_masked_batch(device):
    """Every key of batch 1 masked by the key bias: its rows get O = 0, LSE = -inf
    and zero gradients; batch 0 is ordinary."""
    B, Hq, Hkv, Nq, Nkv, d = 2, 4, 2, 150, 200, 128
    x = inputs.make_custom(13, B, Hq, Hkv, Nq, Nkv, d, "bf16")
    bias = _bias(8, (B, 1, 1, Nkv), Nkv, "bf16")
    bias[1] = float("-inf")
    case = inputs.Case("kb_masked_batch", 0, 0, B, Hq, Hkv, Nq, Nkv, d, "bf16", True, 0.125)
    ref = _oracle(case, x, bias, 0.0, 0, False)
    got = _run(case, x, bias, 0.0, 0, device, False)
    g = _compare(case, got, ref, "masked batch")
    assert np.all(g["o"][1] == 0) and np.all(g["lse"][1] == -np.inf)
    assert np.all(g["dq"][1] == 0) and np.all(g["dk"][1] == 0) and np.all(g["dv"][1] == 0)


@pytest.mark.parametrize("d,dt", [(128, "bf16"), (96, "fp16"), (192, "bf16"), (256, "fp16")])
def test_autograd_key_mask_without_grad(d, dt, device):
    """attention(..., bias=mask) with a key-padding mask that needs no gradient (the
    key-bias instances, built at every head dim) against the oracle: O and the
    gradients in q, k, v."""
    from exact_attention_backward_fa_amd import attention
    B, Hq, Hkv, Nq, Nkv = 2, 8, 2, 257, 384
    x = inputs.make_custom(78 + d, B, Hq, Hkv, Nq, Nkv, d, dt)
    mask = torch.zeros(B, 1, 1, Nkv, dtype=inputs.TORCH_DTYPE[dt])
    mask[0, ..., 300:] = float("-inf")
    mask[1, ..., 17:40] = float("-inf")
    case = inputs.Case("autograd_key_mask", 0, 0, B, Hq, Hkv, Nq, Nkv, d, dt, True, 1.0 / np.sqrt(d))
    ref = _oracle(case, x, mask, 0.0, 0, False)
    q, k, v = (x[n].to(device).requires_grad_() for n in ("q", "k", "v"))
    o = attention(q, k, v, causal=True, bias=mask.to(device))
    (o.float() * x["do"].to(device).float()).sum().backward()
    torch.cuda.synchronize(device)
    got = {"o": o.detach().double().cpu().numpy(), "dq": q.grad.double().cpu().numpy(),
           "dk": k.grad.double().cpu().numpy(), "dv": v.grad.double().cpu().numpy()}
    r = {kk: ref[kk] for kk in ("o", "dq", "dk", "dv")}
    pu.assert_within(case, pu.compare(case, got, r, "autograd key mask"))


def test_dropout_mask_is_the_oracles(device):
    """With V = identity rows and dO = 0, O = (P o Z) V exposes the kept pattern:
    O[i, j] != 0 exactly where the oracle keeps (i, j) (P > 0 everywhere: no bias,
    non-causal).  Compared element for element on one head."""
    B, Hq, Hkv, N, d = 1, 2, 1, 64, 64
    g = torch.Generator().manual_seed(5)
    q = (0.1 * torch.randn(B, Hq, N, d, generator=g)).half()
    k = (0.1 * torch.randn(B, Hkv, N, d, generator=g)).half()
    v = torch.eye(N, d).reshape(1, 1, N, d).half()
    import exact_attention_backward_fa_amd as fa
    seed = 987654321987
    o, _ = fa.fwd_bias_dropout(q.to(device), k.to(device), v.to(device), 0.125, False,
                               dropout_p=0.4, seed=seed)
    torch.cuda.synchronize(device)
    for h in range(Hq):
        z = orc.dropout_factors(0, h, np.arange(N), N, 0.4, seed)
        kept_gpu = o[0, h].float().cpu().numpy() != 0
        assert np.array_equal(kept_gpu, z > 0), f"head {h}: keep pattern differs"


def test_fully_masked_rows(device):
    """Rows whose every key has bias -inf: O = 0, LSE = -inf, zero gradients."""
    import exact_attention_backward_fa_amd as fa
    B, Hq, Hkv, Nq, Nkv, d = 1, 2, 1, 40, 72, 64
    x = inputs.make_custom(11, B, Hq, Hkv, Nq, Nkv, d, "bf16")
    bias = _bias(3, (B, 1, Nq, Nkv), Nkv, "bf16")
    bias[:, :, 5] = float("-inf")
    bias[:, :, 17] = float("-inf")
    case = inputs.Case("masked_rows", 0, 0, B, Hq, Hkv, Nq, Nkv, d, "bf16", False, 0.125)
    ref = _oracle(case, x, bias, 0.0, 0, True)
    got = _run(case, x, bias, 0.0, 0, device, True)
    g = _compare(case, got, ref, "masked rows")
    for r in (5, 17):
        assert np.all(g["o"][:, :, r] == 0) and np.all(g["lse"][:, :, r] == -np.inf)
        assert np.all(g["dq"][:, :, r] == 0) and np.all(g["dbias"][:, :, r] == 0)


def test_dropout_p_one(device):
    """p = 1 drops every element: O = 0 and every gradient 0 (dP o Z = 0 and
    D = rowsum(dO o O) = 0), while LSE stays that of the undropped scores."""
    B, Hq, Hkv, Nq, Nkv, d = 1, 4, 2, 150, 90, 128
    x = inputs.make_custom(21, B, Hq, Hkv, Nq, Nkv, d, "fp16")
    bias = _bias(6, (B, Hq, Nq, Nkv), Nkv, "fp16")
    case = inputs.Case("dropout_p1", 0, 0, B, Hq, Hkv, Nq, Nkv, d, "fp16", True, 1.0 / np.sqrt(d))
    ref = _oracle(case, x, bias, 1.0, 5, True)
    got = _run(case, x, bias, 1.0, 5, device, True)
    for name in ("o", "dq", "dk", "dv", "dbias"):
        assert np.all(ref[name] == 0), name
        assert torch.all(got[name] == 0), name
    lse = got["lse"].double().numpy()
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - ref["lse"][fin]).max() <= 1e-3


RISING_DROP = [(64, False, 0.75, 13), (128, True, 0.9, 12)]


@pytest.mark.parametrize("d,causal,p,h", RISING_DROP, ids=[f"d{c[0]}_p{c[2]}" for c in RISING_DROP])
def test_dropout_fp16_rising_scores(d, causal, p, h, device):
    """fp16 with a high dropout rate and scores that rise about 14 log2 units past
    the first pair of keys.  The forward rounds P o Z to fp16 for the P V product,
    with Z = 256 / T up to 4 (p = 0.75) or 9.8 (p = 0.9), so a P below the plain
    headroom 2^15 could still round to inf once scaled; the headroom drops to h
    (the largest with 2^h Z < 65520), and items past it rerun with raised
    references.  O, LSE and the gradients must be finite and match the oracle."""
    B, Hq, Hkv, N = 1, 2, 1, 384
    g = torch.Generator().manual_seed(4545)
    u = torch.full((d,), 1.0 / np.sqrt(d))
    ramp = torch.arange(N, dtype=torch.float32) / N
    amp = 10.8 / 5.0
    x = {
        "q": (5.0 * u + 0.02 * torch.randn(B, Hq, N, d, generator=g)).half(),
        "k": (amp * ramp[:, None] * u + 0.02 * torch.randn(B, Hkv, N, d, generator=g)).half(),
        "v": torch.randn(B, Hkv, N, d, generator=g).half(),
        "do": torch.randn(B, Hq, N, d, generator=g).half(),
    }
    t = int(np.floor((1.0 - p) * 256 + 0.5))
    assert 2.0 ** h * 256 / t < 65520 <= 2.0 ** (h + 1) * 256 / t
    # the premise: visible scores more than h but less than 15 log2 units past the
    # maximum over the first 32 keys, in some rows (causal) or all
    sc = orc.as_f64(x["q"][0]) @ orc.as_f64(x["k"][0, 0]).T / np.log(2.0)
    rows = range(32, N)
    over = np.array([[sc[hh, r, 32:(r + 1 if causal else N)].max() - sc[hh, r, :32].max() for r in rows]
                     for hh in range(Hq)])
    assert over.max() < 15.0 and (over > h).mean() > (0.1 if causal else 0.9)
    case = inputs.Case(f"rising_drop_d{d}", 0, 0, B, Hq, Hkv, N, N, d, "fp16", causal, 1.0)
    ref = _oracle(case, x, None, p, 99, False)
    got = _run(case, x, None, p, 99, device, False)
    assert all(bool(torch.isfinite(got[k]).all()) for k in ("o", "dq", "dk", "dv"))
    _compare(case, got, ref, case.name)


@pytest.mark.parametrize("what", ["dropout", "key_mask"])
def test_headline_shape_features_sampled(what, device):
    """The full headline workload (causal GQA B=4 Hq=32 Hkv=8 N=8192 d=128 bf16)
    through the feature entry points, as `bench.py --dropout 0.1` (seed 77) and
    `bench.py --bias keys` (the last eighth of the keys masked) run it.  Compared
    with the oracle's row functions under the same mask or bias: 32 query rows
    (O, LSE, dQ) of the first and the last head, and key rows (dK, dV) of the first
    and last kv head: the trailing 48, and for the first also the leading 64, whose
    sums run over every query row of the group."""
    case = inputs.case_by_name(inputs.HEADLINE)
    x = inputs.make_inputs(case)
    N = case.Nkv
    if what == "dropout":
        bias, p, seed = None, 0.1, 77
    else:
        store = torch.zeros(case.B, 1, 1, (N + 7) // 8 * 8, dtype=case.torch_dtype)
        store[..., N - N // 8:] = float("-inf")
        bias, p, seed = store[..., :N], 0.0, 0
    pu.log(f"[gpu] headline shape, {what}")
    got = _run(case, x, bias, p, seed, device, False)
    extras = {"bias": None if bias is None else orc.as_f64(bias), "dropout_p": p, "seed": seed}
    rng = np.random.default_rng(2024)
    rows = np.unique(np.concatenate([[0, 1, N // 2, N - 2, N - 1], rng.integers(0, N, 27)]))
    tail = np.arange(N - 48, N)
    for n, (b, h, g) in enumerate([(0, 0, 0), (case.B - 1, case.Hq - 1, case.Hkv - 1)]):
        kv_rows = np.concatenate([np.arange(64), tail]) if n == 0 else tail
        pu.log(f"[oracle] rows b={b} h={h} g={g} ({len(kv_rows)} key rows)")
        o, l_ = orc.forward_rows(x["q"], x["k"], x["v"], case.scale, case.causal, b, h, rows, **extras)
        dq = orc.dq_rows(x["q"], x["k"], x["v"], x["do"], case.scale, case.causal, b, h, rows,
                         **extras)
        dk, dv = pu.dkdv_rows_by_head(case, x, b, g, kv_rows, **extras)
        ref = {"o": o, "lse": l_, "dq": dq, "dk": dk, "dv": dv}
        sub = {"o": got["o"][b, h, rows], "lse": got["lse"][b, h, rows], "dq": got["dq"][b, h, rows],
               "dk": got["dk"][b, g, kv_rows], "dv": got["dv"][b, g, kv_rows]}
        _compare(case, sub, ref, f"{what} rows b={b} h={h}")


def test_long_sequence_bias_dropout(device):
    """N = 2048 causal GQA bf16 with a full bias and dropout: several work items per
    head in every kernel; every head compared."""
    B, Hq, Hkv, N, d = 1, 8, 2, 2048, 128
    x = inputs.make_custom(2048, B, Hq, Hkv, N, N, d, "bf16")
    case = inputs.Case("long_bias_dropout", 0, 0, B, Hq, Hkv, N, N, d, "bf16", True, 1.0 / np.sqrt(d))
    bias = _bias(9, (B, Hq, N, N), N, "bf16", mult=1.0)
    ref = _oracle(case, x, bias, 0.15, 42, False)
    got = _run(case, x, bias, 0.15, 42, device, False)
    _compare(case, got, ref, "all heads")


def test_autograd_bias_and_dropout(device):
    """attention(..., bias=, dropout_p=, seed=) against the oracle: O, and the
    gradients of <O, dO> in q, k, v and a bias broadcast over the heads (its
    gradient is dBias summed over the heads)."""
    from exact_attention_backward_fa_amd import attention
    B, Hq, Hkv, Nq, Nkv, d = 2, 4, 2, 130, 200, 64
    x = inputs.make_custom(77, B, Hq, Hkv, Nq, Nkv, d, "bf16")
    bias = _bias(4, (B, 1, Nq, Nkv), Nkv, "bf16")
    case = inputs.Case("autograd_bias", 0, 0, B, Hq, Hkv, Nq, Nkv, d, "bf16", True, 1.0 / np.sqrt(d))
    ref = _oracle(case, x, bias, 0.25, 99, True)
    q, k, v = (x[n].to(device).requires_grad_() for n in ("q", "k", "v"))
    bd = _bias_to(bias, device).detach().requires_grad_()
    o = attention(q, k, v, causal=True, bias=bd, dropout_p=0.25, seed=99)
    (o.float() * x["do"].to(device).float()).sum().backward()
    torch.cuda.synchronize(device)
    got = {"o": o.detach().double().cpu().numpy(), "dq": q.grad.double().cpu().numpy(),
           "dk": k.grad.double().cpu().numpy(), "dv": v.grad.double().cpu().numpy()}
    r = {kk: ref[kk] for kk in ("o", "dq", "dk", "dv")}
    pu.assert_within(case, pu.compare(case, got, r, "autograd"))
    db_ref = ref["dbias"].sum(axis=1, keepdims=True)
    err = pu.rel_err(bd.grad.double().cpu().numpy(), db_ref)
    pu.log(f"  autograd dbias (summed over heads) {err:.2e}")
    assert err <= pu.TOL["bf16"]


def test_rejected_extras(device):
    import exact_attention_backward_fa_amd as fa
    x = pu.to_dev(inputs.make_custom(1, 1, 2, 1, 64, 64, 96, "fp16"), device)
    with pytest.raises(RuntimeError, match="status -3"):   # bias/dropout need d = 64 or 128
        fa.fwd_bias_dropout(x["q"], x["k"], x["v"], 0.1, False, dropout_p=0.1)
    x = pu.to_dev(inputs.make_custom(1, 1, 2, 1, 64, 64, 64, "fp16"), device)
    with pytest.raises(RuntimeError, match="status -12"):
        fa.fwd_bias_dropout(x["q"], x["k"], x["v"], 0.1, False, dropout_p=1.5)
