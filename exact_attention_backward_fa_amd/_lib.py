"""ctypes binding of libfa_mi355x.so.

Argument marshalling only: every step of the attention computation runs in the
HIP kernels behind the C ABI.  torch supplies device memory and the stream.
There is no fallback: if the library is missing or a call fails, this raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa_mi355x.so")

FA_DTYPE = {torch.float16: 0, torch.bfloat16: 1}
DQ_MODES = {"auto": 0, "atomic": 1, "separate": 2}
DQ_MODE_NAMES = {v: k for k, v in DQ_MODES.items()}

# Names the header declares; the CPU tests check the library exports each one.
EXPORTS = (
    "fa_fwd", "fa_bwd", "fa_bwd_ex", "fa_bwd_workspace_bytes",
    "fa_bwd_ex_workspace_bytes", "fa_bwd_auto_dq_mode", "fa_status_string", "fa_version",
    "fa_bwd_noalloc", "fa_bwd_noalloc_max_scratch_bytes", "fa_fwd_bias_dropout",
    "fa_bwd_bias_dropout",
)

_lib = None

_i, _f, _p, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_ll, _ull = ctypes.c_longlong, ctypes.c_ulonglong


def load() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m exact_attention_backward_fa_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_fwd.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _p]
    lib.fa_fwd.restype = _i
    lib.fa_bwd.argtypes = [_p] * 9 + [_i] * 6 + [_f, _i, _i, _p, _sz, _p]
    lib.fa_bwd.restype = _i
    lib.fa_bwd_ex.argtypes = [_p] * 9 + [_i] * 6 + [_f, _i, _i, _i, _p, _p, _p, _sz, _p]
    lib.fa_bwd_ex.restype = _i
    lib.fa_bwd_workspace_bytes.argtypes = [_i] * 8
    lib.fa_bwd_workspace_bytes.restype = _sz
    lib.fa_bwd_ex_workspace_bytes.argtypes = [_i] * 9
    lib.fa_bwd_ex_workspace_bytes.restype = _sz
    lib.fa_bwd_auto_dq_mode.argtypes = [_i] * 8
    lib.fa_bwd_auto_dq_mode.restype = _i
    lib.fa_status_string.argtypes = [_i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = _i
    lib.fa_bwd_noalloc.argtypes = [_p] * 9 + [_i] * 6 + [_f, _i, _i, _p]
    lib.fa_bwd_noalloc.restype = _i
    lib.fa_bwd_noalloc_max_scratch_bytes.argtypes = []
    lib.fa_bwd_noalloc_max_scratch_bytes.restype = _sz
    lib.fa_fwd_bias_dropout.argtypes = ([_p] * 5 + [_i] * 6 + [_f, _i, _i, _p, _ll, _ll, _ll, _f, _ull,
                                                                _p])
    lib.fa_fwd_bias_dropout.restype = _i
    lib.fa_bwd_bias_dropout.argtypes = ([_p] * 9 + [_i] * 6 + [_f, _i, _i, _p, _ll, _ll, _ll, _p, _f,
                                                                _ull, _p, _sz, _p])
    lib.fa_bwd_bias_dropout.restype = _i
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().fa_status_string(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise RuntimeError(f"{what} failed: status {code} ({status_string(code)})")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _shapes(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nkv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError(f"shape mismatch q={tuple(q.shape)} k={tuple(k.shape)} v={tuple(v.shape)}")
    return B, Hq, Hkv, Nq, Nkv, d


def _check_tensors(dtype: torch.dtype, device: torch.device, **ts) -> None:
    if dtype not in FA_DTYPE:
        raise ValueError(f"dtype must be float16 or bfloat16, got {dtype}")
    if device.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t in ts.items():
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def fwd_into(q, k, v, o, lse, scale: float, causal: bool) -> None:
    """Forward into preallocated o [B,Hq,Nq,d] and lse [B,Hq,Nq] float32."""
    B, Hq, Hkv, Nq, Nkv, d = _shapes(q, k, v)
    _check_tensors(q.dtype, q.device, q=q, k=k, v=v, o=o, lse=lse)
    if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype or lse.dtype != torch.float32:
        raise ValueError("dtype mismatch")
    if tuple(o.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("output shape mismatch")
    lib = load()
    _check(lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nkv, d,
                      float(scale), int(bool(causal)), FA_DTYPE[q.dtype], _stream(q.device)),
           "fa_fwd")


def fwd(q, k, v, scale: float, causal: bool) -> Tuple[torch.Tensor, torch.Tensor]:
    """Returns (o, lse): o like q, lse float32 [B, Hq, Nq] (natural log)."""
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fwd_into(q, k, v, o, lse, scale, causal)
    return o, lse


def bwd_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, causal, dtype, dq_mode: str = "auto") -> int:
    return int(load().fa_bwd_ex_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, int(bool(causal)),
                                                FA_DTYPE[dtype], DQ_MODES[dq_mode]))


def auto_dq_mode(B, Hq, Hkv, Nq, Nkv, d, causal, dtype) -> str:
    m = load().fa_bwd_auto_dq_mode(B, Hq, Hkv, Nq, Nkv, d, int(bool(causal)), FA_DTYPE[dtype])
    return DQ_MODE_NAMES[m]


def bwd_into(q, k, v, o, lse, do, dq, dk, dv, scale: float, causal: bool, *,
             dq_mode: str = "auto", workspace: Optional[torch.Tensor] = None,
             events: Optional[Tuple[int, int]] = None) -> None:
    """Backward into preallocated dq, dk, dv.  ``workspace`` (uint8, on device)
    is allocated here when not given.  ``events``: optional pair of raw hipEvent_t
    handles recorded around the dK/dV kernel."""
    B, Hq, Hkv, Nq, Nkv, d = _shapes(q, k, v)
    _check_tensors(q.dtype, q.device, q=q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv)
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} != q dtype {q.dtype}")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("lse must be float32 [B, Hq, Nq]")
    for name, t, ref in (("o", o, q), ("do", do, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(ref.shape)}")
    if dq_mode not in DQ_MODES:
        raise ValueError(f"dq_mode must be one of {list(DQ_MODES)}")
    need = bwd_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, causal, q.dtype, dq_mode)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ev0, ev1 = (None, None) if events is None else events
    lib = load()
    _check(lib.fa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                         _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, Nkv, d, float(scale),
                         int(bool(causal)), FA_DTYPE[q.dtype], DQ_MODES[dq_mode], ev0, ev1,
                         _ptr(workspace), workspace.numel(), _stream(q.device)),
           "fa_bwd_ex")


def bwd(q, k, v, o, lse, do, scale: float, causal: bool, *, dq_mode: str = "auto"):
    """Returns (dq, dk, dv) in the input dtype."""
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    bwd_into(q, k, v, o, lse, do, dq, dk, dv, scale, causal, dq_mode=dq_mode)
    return dq, dk, dv


# --- additive score bias and dropout ------------------------------------------

def _bias_args(bias, q, k):
    """(pointer, stride_b, stride_h, stride_q) of a bias broadcastable to
    [B, Hq, Nq, Nkv] (a 4-D tensor whose dimensions are those sizes or 1, key
    dimension contiguous), or (None, 0, 0, 0)."""
    if bias is None:
        return None, 0, 0, 0
    B, Hq, Nq, _ = q.shape
    Nkv = k.shape[2]
    if bias.dim() != 4 or bias.dtype != q.dtype or bias.device != q.device:
        raise ValueError("bias must be a 4-D tensor of q's dtype on q's device")
    want = (B, Hq, Nq, Nkv)
    for got, full in zip(bias.shape, want):
        if got not in (1, full):
            raise ValueError(f"bias shape {tuple(bias.shape)} does not broadcast to {want}")
    if bias.shape[3] != Nkv or (Nkv > 1 and bias.stride(3) != 1):
        raise ValueError("bias must span N_kv keys with the key dimension contiguous")
    strides = [0 if bias.shape[i] == 1 else bias.stride(i) for i in range(3)]
    if any(st % 8 for st in strides) or bias.data_ptr() % 16:
        raise ValueError("bias rows must be 16-byte aligned (strides multiples of 8 elements); "
                         "pad the key dimension of the storage to a multiple of 8")
    # the kernels read each row in whole 16-byte pieces: N_kv rounded up to 8 elements
    last = sum((bias.shape[i] - 1) * strides[i] for i in range(3)) + (Nkv + 7) // 8 * 8
    end = bias.storage_offset() + last
    if end * bias.element_size() > bias.untyped_storage().nbytes():
        raise ValueError("each bias row must be readable for N_kv rounded up to a multiple of 8 "
                         "elements: pad the key dimension of the storage")
    return bias.data_ptr(), strides[0], strides[1], strides[2]


def fwd_bias_dropout(q, k, v, scale: float, causal: bool, *, bias=None, dropout_p: float = 0.0,
                     seed: int = 0, o=None, lse=None):
    """fa_fwd_bias_dropout: returns (o, lse).  ``bias`` broadcasts to [B, Hq, Nq, Nkv]."""
    B, Hq, Hkv, Nq, Nkv, d = _shapes(q, k, v)
    _check_tensors(q.dtype, q.device, q=q, k=k, v=v)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensors(q.dtype, q.device, o=o, lse=lse)
    bp, sb, sh, sq = _bias_args(bias, q, k)
    lib = load()
    _check(lib.fa_fwd_bias_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq,
                                   Nkv, d, float(scale), int(bool(causal)), FA_DTYPE[q.dtype], bp,
                                   sb, sh, sq, float(dropout_p), int(seed) & (2 ** 64 - 1),
                                   _stream(q.device)),
           "fa_fwd_bias_dropout")
    return o, lse


def bwd_bias_dropout(q, k, v, o, lse, do, scale: float, causal: bool, *, bias=None,
                     want_dbias: bool = False, dropout_p: float = 0.0, seed: int = 0,
                     dq=None, dk=None, dv=None, dbias=None, workspace=None):
    """fa_bwd_bias_dropout: returns (dq, dk, dv, dbias or None); dbias is the full
    [B, Hq, Nq, Nkv] gradient of the scores' bias.  Outputs and the workspace may be
    passed in (then nothing is allocated); a given ``dbias`` implies want_dbias."""
    B, Hq, Hkv, Nq, Nkv, d = _shapes(q, k, v)
    _check_tensors(q.dtype, q.device, q=q, k=k, v=v, o=o, lse=lse, do=do)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dbias is None and want_dbias:
        dbias = torch.empty((B, Hq, Nq, Nkv), dtype=q.dtype, device=q.device)
    _check_tensors(q.dtype, q.device, dq=dq, dk=dk, dv=dv)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq, dk, dv must have the shapes of q, k, v")
    if any(t is not None and t.dtype != q.dtype for t in (dq, dk, dv, dbias)):
        raise ValueError("dq, dk, dv and dbias must have q's dtype")
    if dbias is not None:
        _check_tensors(q.dtype, q.device, dbias=dbias)
        if tuple(dbias.shape) != (B, Hq, Nq, Nkv):
            raise ValueError(f"dbias must be [B, Hq, Nq, Nkv] = {(B, Hq, Nq, Nkv)}")
    bp, sb, sh, sq = _bias_args(bias, q, k)
    need = bwd_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, causal, q.dtype, "separate")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device) if workspace is None else workspace
    lib = load()
    _check(lib.fa_bwd_bias_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                   _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, Nkv, d, float(scale),
                                   int(bool(causal)), FA_DTYPE[q.dtype], bp, sb, sh, sq,
                                   _ptr(dbias), float(dropout_p), int(seed) & (2 ** 64 - 1),
                                   _ptr(ws), ws.numel(), _stream(q.device)),
           "fa_bwd_bias_dropout")
    return dq, dk, dv, dbias


# --- raw HIP events (timing on the exact stream the kernels run on) -------------

_hip = None


def _hip_rt() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise RuntimeError("libamdhip64.so not found")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _p, _p]
        _hip.hipEventSynchronize.argtypes = [_p]
        _hip.hipEventDestroy.argtypes = [_p]
        _hip.hipEventRecord.argtypes = [_p, _p]
    return _hip


class HipEvent:
    """A plain hipEvent_t (timing enabled) owned by Python."""

    def __init__(self):
        h = ctypes.c_void_p()
        rc = _hip_rt().hipEventCreate(ctypes.byref(h))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        self.handle = h.value

    def record(self, stream: int) -> None:
        rc = _hip_rt().hipEventRecord(self.handle, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def synchronize(self) -> None:
        _hip_rt().hipEventSynchronize(self.handle)

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = _hip_rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle:
                _hip_rt().hipEventDestroy(self.handle)
        except Exception:
            pass
