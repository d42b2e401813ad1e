"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before touching a device.

No call here passes a valid set of arguments, so nothing is ever launched.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")

FA_OK, FA_ERR_NULLPTR, FA_ERR_SHAPE, FA_ERR_HEADDIM = 0, -1, -2, -3
FA_ERR_DTYPE, FA_ERR_SCALE, FA_ERR_WORKSPACE, FA_ERR_ALIGN, FA_ERR_HIP, FA_ERR_MODE = -4, -5, -6, -7, -8, -9
FA_ERR_SCRATCH, FA_ERR_BIAS, FA_ERR_DROPOUT = -10, -11, -12


@pytest.fixture(scope="module")
def lib():
    from exact_attention_backward_fa_amd import _lib
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_api():
    names = header_functions()
    from exact_attention_backward_fa_amd import _lib
    assert sorted(_lib.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    from exact_attention_backward_fa_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_[a-z_0-9]+)\b", out))
    for name in header_functions():
        assert name in exported, f"{name} not exported"
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code in (FA_OK, FA_ERR_NULLPTR, FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_DTYPE, FA_ERR_SCALE,
                 FA_ERR_WORKSPACE, FA_ERR_ALIGN, FA_ERR_HIP, FA_ERR_MODE, FA_ERR_SCRATCH, FA_ERR_BIAS,
                 FA_ERR_DROPOUT, 12345):
        s = lib.fa_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.fa_status_string(FA_ERR_HEADDIM).decode().find("96") >= 0
    assert lib.fa_version() >= 100


# Fake, 16-byte aligned, never dereferenced addresses: every call below fails
# validation before anything reads them.
P = 0x10000


def fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nkv=8, d=64, scale=0.125,
             causal=0, dtype=0)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                      a["Nkv"], a["d"], a["scale"], a["causal"], a["dtype"], None)


def bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=1, Nq=8, Nkv=8,
             d=64, scale=0.125, causal=0, dtype=0, mode=0, ws=P, wsb=1 << 40)
    a.update(kw)
    return lib.fa_bwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                         a["dv"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["d"], a["scale"],
                         a["causal"], a["dtype"], a["mode"], None, None, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("call", [fwd, bwd])
def test_argument_errors(lib, call):
    assert call(lib, dtype=2) == FA_ERR_DTYPE
    assert call(lib, dtype=-1) == FA_ERR_DTYPE
    for d in (0, 8, 16, 48, 80, 112, 200, 288, 512, -64):
        assert call(lib, d=d) == FA_ERR_HEADDIM, d
    assert call(lib, Hq=3, Hkv=2) == FA_ERR_SHAPE
    assert call(lib, Hkv=0) == FA_ERR_SHAPE
    assert call(lib, Hq=0) == FA_ERR_SHAPE
    assert call(lib, B=-1) == FA_ERR_SHAPE
    assert call(lib, Nq=-5) == FA_ERR_SHAPE
    assert call(lib, Nkv=-1) == FA_ERR_SHAPE
    assert call(lib, Nq=1 << 25, d=128) == FA_ERR_SHAPE  # N*d >= 2^31
    assert call(lib, B=70000) == FA_ERR_SHAPE
    assert call(lib, scale=0.0) == FA_ERR_SCALE
    assert call(lib, scale=-1.0) == FA_ERR_SCALE
    assert call(lib, scale=math.inf) == FA_ERR_SCALE
    assert call(lib, scale=math.nan) == FA_ERR_SCALE
    assert call(lib, q=0) == FA_ERR_NULLPTR
    assert call(lib, q=P + 8) == FA_ERR_ALIGN
    assert call(lib, lse=P + 4) == FA_ERR_ALIGN


def test_bwd_specific_errors(lib):
    for name in ("o", "do", "dq", "dk", "dv", "k", "v"):
        assert bwd(lib, **{name: 0}) == FA_ERR_NULLPTR, name
        assert bwd(lib, **{name: P + 2}) == FA_ERR_ALIGN, name
    assert bwd(lib, mode=3) == FA_ERR_MODE
    assert bwd(lib, mode=-1) == FA_ERR_MODE
    assert bwd(lib, ws=0) == FA_ERR_WORKSPACE
    assert bwd(lib, ws=P + 8) == FA_ERR_WORKSPACE
    need = lib.fa_bwd_ex_workspace_bytes(1, 2, 1, 8, 8, 64, 0, 0, 1)
    assert need > 0
    assert bwd(lib, mode=1, wsb=need - 1) == FA_ERR_WORKSPACE
    need_sep = lib.fa_bwd_ex_workspace_bytes(1, 2, 1, 8, 8, 64, 0, 0, 2)
    assert bwd(lib, mode=2, wsb=need_sep - 1) == FA_ERR_WORKSPACE


def test_head_dims_and_the_atomic_path(lib):
    """Every multiple of 32 up to 256 is accepted (the call here then stops at the
    workspace check); the fused atomic dQ kernel exists for 64 and 128 only."""
    for d in (32, 64, 96, 128, 160, 192, 224, 256):
        assert bwd(lib, d=d, mode=2, ws=0) == FA_ERR_WORKSPACE, d
        assert fwd(lib, d=d, q=0) == FA_ERR_NULLPTR, d
        assert lib.fa_bwd_ex_workspace_bytes(1, 2, 1, 8, 8, d, 0, 0, 2) > 0
        atomic_ws = lib.fa_bwd_ex_workspace_bytes(1, 2, 1, 8, 8, d, 0, 0, 1)
        if d in (64, 128):
            assert atomic_ws > 0
            assert bwd(lib, d=d, mode=1, ws=0) == FA_ERR_WORKSPACE
        else:
            assert atomic_ws == 0
            assert bwd(lib, d=d, mode=1) == FA_ERR_HEADDIM
    assert b"256" in lib.fa_status_string(FA_ERR_HEADDIM)


def test_workspace_sizes(lib):
    B, Hq, Hkv, N, d = 4, 32, 8, 8192, 128
    rows = B * Hq * N
    atomic = lib.fa_bwd_ex_workspace_bytes(B, Hq, Hkv, N, N, d, 1, 1, 1)
    separate = lib.fa_bwd_ex_workspace_bytes(B, Hq, Hkv, N, N, d, 1, 1, 2)
    assert separate >= 2 * rows * 4 and separate < 2 * rows * 4 + 1024
    assert atomic >= separate + rows * d * 4
    auto = lib.fa_bwd_workspace_bytes(B, Hq, Hkv, N, N, d, 1, 1)
    assert auto in (atomic, separate)
    mode = lib.fa_bwd_auto_dq_mode(B, Hq, Hkv, N, N, d, 1, 1)
    assert mode in (1, 2)
    assert auto == (atomic if mode == 1 else separate)
    # zero-size problems need no workspace; invalid ones report 0
    assert lib.fa_bwd_workspace_bytes(0, Hq, Hkv, N, N, d, 1, 1) == 0
    assert lib.fa_bwd_workspace_bytes(B, Hq, Hkv, 0, N, d, 1, 1) == 0
    assert lib.fa_bwd_workspace_bytes(B, 3, 2, N, N, d, 1, 1) == 0
    assert lib.fa_bwd_ex_workspace_bytes(B, Hq, Hkv, N, N, d, 1, 1, 7) == 0


def test_null_pointers_allowed_for_empty_tensors_only(lib):
    # N_q = 0: q/o/lse/do/dq are empty, so NULL is accepted for them, but dk still
    # has elements (it is written with zeros), so a NULL dk is rejected.
    assert bwd(lib, Nq=0, q=0, o=0, lse=0, do=0, dq=0, dk=0) == FA_ERR_NULLPTR
    # forward with B = 0 touches nothing at all: every pointer may be NULL and the
    # call succeeds without enqueuing work.
    assert fwd(lib, B=0, q=0, k=0, v=0, o=0, lse=0) == FA_OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    import exact_attention_backward_fa_amd as fa
    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q, 0.125, False)
    with pytest.raises(ValueError):
        fa.fwd(q.float(), q.float(), q.float(), 0.125, False)


def noalloc(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=1, Nq=8, Nkv=8,
             d=64, scale=0.125, causal=0, dtype=0)
    a.update(kw)
    return lib.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                              a["dv"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["d"],
                              a["scale"], a["causal"], a["dtype"], None)


def test_noalloc_checks_arguments_before_any_device_call(lib):
    """fa_bwd_noalloc applies fa_bwd's checks, and rejects a problem whose scratch
    exceeds its static array, before it touches a device (none exists here)."""
    cap = lib.fa_bwd_noalloc_max_scratch_bytes()
    assert cap == 16 << 20
    assert b"scratch" in lib.fa_status_string(FA_ERR_SCRATCH)
    assert noalloc(lib, d=80) == FA_ERR_HEADDIM
    assert noalloc(lib, Hq=3, Hkv=2) == FA_ERR_SHAPE
    assert noalloc(lib, scale=-1.0) == FA_ERR_SCALE
    assert noalloc(lib, dtype=5) == FA_ERR_DTYPE
    assert noalloc(lib, dq=0) == FA_ERR_NULLPTR
    assert noalloc(lib, dv=P + 2) == FA_ERR_ALIGN
    # the largest problem that fits, and one query row per head more than that
    sep = lambda B, Hq, N: lib.fa_bwd_ex_workspace_bytes(B, Hq, 1, N, N, 64, 0, 0, 2)
    n = 1
    while sep(1, 1, 2 * n) <= cap:
        n *= 2
    lo, hi = n, 2 * n
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if sep(1, 1, mid) <= cap else (lo, mid)
    assert sep(1, 1, lo) <= cap < sep(1, 1, lo + 1)
    assert noalloc(lib, Hq=1, Nq=lo + 1, Nkv=16) == FA_ERR_SCRATCH
    assert noalloc(lib, B=4, Hq=32, Hkv=8, Nq=32768, Nkv=32768, d=128, causal=1,
                   dtype=1) == FA_ERR_SCRATCH


def fwd_bd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nkv=8, d=64, scale=0.125,
             causal=0, dtype=0, bias=P, sb=0, sh=0, sq=8, p=0.0, seed=1)
    a.update(kw)
    return lib.fa_fwd_bias_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                   a["Nq"], a["Nkv"], a["d"], a["scale"], a["causal"], a["dtype"],
                                   a["bias"], a["sb"], a["sh"], a["sq"], a["p"], a["seed"], None)


def bwd_bd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=1, Nq=8, Nkv=8,
             d=64, scale=0.125, causal=0, dtype=0, bias=P, sb=0, sh=0, sq=8, dbias=P, p=0.0, seed=1,
             ws=0, wsb=0)
    a.update(kw)
    return lib.fa_bwd_bias_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                   a["dv"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["d"],
                                   a["scale"], a["causal"], a["dtype"], a["bias"], a["sb"], a["sh"],
                                   a["sq"], a["dbias"], a["p"], a["seed"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("call", [fwd_bd, bwd_bd])
def test_bias_dropout_argument_errors(lib, call):
    """Checked on the host before any device call (none exists here)."""
    for p in (-0.01, 1.01, math.nan, math.inf):
        assert call(lib, p=p) == FA_ERR_DROPOUT, p
    assert call(lib, sq=4) == FA_ERR_BIAS        # rows not 16-byte aligned
    assert call(lib, sq=-8) == FA_ERR_BIAS
    assert call(lib, sh=12) == FA_ERR_BIAS
    assert call(lib, sq=(1 << 22) + 8) == FA_ERR_BIAS
    assert call(lib, bias=P + 8) == FA_ERR_ALIGN
    assert call(lib, d=96) == FA_ERR_HEADDIM     # a bias along rows needs d = 64 or 128
    # a bias per (batch, key) without dBias runs at every head dim: the call goes on
    # to the pointer checks
    kb = {"sq": 0, "q": 0, **({"dbias": 0} if call is bwd_bd else {})}
    for d in (32, 96, 160, 192, 224, 256):
        assert call(lib, d=d, **kb) == FA_ERR_NULLPTR, d
    assert call(lib, d=96, p=0.1, **kb) == FA_ERR_HEADDIM  # dropout needs d = 64 or 128
    assert call(lib, d=96, bias=0, p=0.5) == FA_ERR_HEADDIM
    assert call(lib, d=96, bias=0, sq=3, p=0.0, **({"dbias": 0} if call is bwd_bd else {})) != FA_ERR_HEADDIM
    assert call(lib, q=0) == FA_ERR_NULLPTR
    assert call(lib, scale=0.0) == FA_ERR_SCALE


def test_bias_dropout_backward_specific_errors(lib):
    assert bwd_bd(lib, dbias=P + 4) == FA_ERR_ALIGN
    # valid arguments stop at the workspace check (separate dQ path sizes)
    assert bwd_bd(lib) == FA_ERR_WORKSPACE
    assert bwd_bd(lib, p=0.3, bias=0, dbias=0) == FA_ERR_WORKSPACE
    # without bias, dbias and dropout the call is the plain backward
    assert bwd_bd(lib, d=96, bias=0, dbias=0) == FA_ERR_WORKSPACE
