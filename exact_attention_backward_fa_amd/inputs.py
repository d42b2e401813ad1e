"""Seeded synthetic workloads shared by the HIP path's tests, the benchmark and
the oracle's tests.

This module only draws random numbers and describes shapes.  It holds none of
the attention arithmetic, so both sides of a parity comparison can take their
inputs from it without sharing any of the method.

Workloads (all synthetic; no dataset is involved):

* ``single``   - one head, B=1, N_q=N_kv=128, d=64, fp16, non-causal, scale 1/8,
  N(0,1) values.  O and LSE handed to the backward come from the oracle's
  forward.
* ``ragged``   - B=2, H=4, d=64, fp16, (N_q, N_kv) in (1,37), (17,17),
  (100,333), (1000,1000), each causal then non-causal, N(0,1) values.  A
  single-row query is the inference case whose failure below one tile is
  reported in the flash-attention-minimal thread "Implement backward pass".
* ``uniform``  - B=2, H=16, N=2048, d=128, fp16, non-causal, scale 1.1,
  U[0,1) values: the shape and value law of the harness in the Triton issue
  "Extra transposes cause 8x speedup for sequence-parallel Flash Attention
  backward".
* ``llama_gqa`` - B=4, Hq=32, Hkv=8, d=128, causal, scale 1/sqrt(128), N(0,1),
  N = 2^5 .. 2^14, fp16 and bf16: the Llama-3 shape of the benchmark section in
  the Liger-Kernel pull request "[Kernel] Flash attention 2".
* ``long_gqa`` - B=1, Hq=32, Hkv=8, N=32768, d=128, bf16, causal, Q and K drawn
  as 2*N(0,1) to sharpen the softmax, V and dO N(0,1); plus a d=64 variant with
  Hq=Hkv=16, N=8192 under the same value law.

Seeds are ``1000*family + sub-case`` (family 1..5 in the order above, sub-cases
counted from 0 in the listed order).  One CPU ``torch.Generator`` per case
draws Q, K, V, dO in that order as fp32, applies the multiplier, then rounds to
the case dtype with round-to-nearest-even.  Both sides receive the rounded
values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List

import torch

FP16 = "fp16"
BF16 = "bf16"

TORCH_DTYPE = {FP16: torch.float16, BF16: torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Case:
    name: str
    family: int
    sub: int
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    d: int
    dtype: str
    causal: bool
    scale: float
    dist: str = "normal"          # "normal" -> N(0,1), "uniform" -> U[0,1)
    qk_mult: float = 1.0          # multiplier applied to Q and K after drawing
    o_lse_from_oracle: bool = False

    @property
    def seed(self) -> int:
        return 1000 * self.family + self.sub

    @property
    def torch_dtype(self) -> torch.dtype:
        return TORCH_DTYPE[self.dtype]

    def bwd_flops(self) -> float:
        """Backward work as the metric counts it: 2.5 x the forward's 4*Nq*Nkv*d
        per query head, halved for causal."""
        f = 2.5 * 4.0 * self.B * self.Hq * self.Nq * self.Nkv * self.d
        return f * (0.5 if self.causal else 1.0)

    def fwd_flops(self) -> float:
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nkv * self.d
        return f * (0.5 if self.causal else 1.0)


def _single() -> List[Case]:
    return [Case("single", 1, 0, 1, 1, 1, 128, 128, 64, FP16, False, 1.0 / 8.0,
                 o_lse_from_oracle=True)]


def _ragged() -> List[Case]:
    out = []
    sub = 0
    for nq, nkv in ((1, 37), (17, 17), (100, 333), (1000, 1000)):
        for causal in (True, False):
            out.append(Case(f"ragged_{nq}x{nkv}_{'c' if causal else 'nc'}", 2, sub,
                            2, 4, 4, nq, nkv, 64, FP16, causal, 1.0 / 8.0))
            sub += 1
    return out


def _uniform() -> List[Case]:
    return [Case("uniform", 3, 0, 2, 16, 16, 2048, 2048, 128, FP16, False, 1.1,
                 dist="uniform")]


def _llama() -> List[Case]:
    out = []
    for lg in range(5, 15):
        n = 1 << lg
        for is_bf16 in (0, 1):
            sub = 2 * (lg - 5) + is_bf16
            dt = BF16 if is_bf16 else FP16
            out.append(Case(f"llama_gqa_{dt}_{n}", 4, sub, 4, 32, 8, n, n, 128, dt,
                            True, 1.0 / math.sqrt(128.0)))
    return out


def _long() -> List[Case]:
    return [
        Case("long_gqa_32768", 5, 0, 1, 32, 8, 32768, 32768, 128, BF16, True,
             1.0 / math.sqrt(128.0), qk_mult=2.0),
        Case("long_d64_8192", 5, 1, 1, 16, 16, 8192, 8192, 64, BF16, True,
             1.0 / math.sqrt(64.0), qk_mult=2.0),
    ]


def all_cases() -> List[Case]:
    return _single() + _ragged() + _uniform() + _llama() + _long()


def case_by_name(name: str) -> Case:
    for c in all_cases():
        if c.name == name:
            return c
    raise KeyError(name)


def cases_of_family(family: int) -> List[Case]:
    return [c for c in all_cases() if c.family == family]


# The workload the headline figure is measured on: Llama-3-style causal GQA,
# B=4, Hq=32, Hkv=8, N=8192, d=128, bf16.
HEADLINE = "llama_gqa_bf16_8192"


def make_inputs(case: Case, *, B: int | None = None) -> Dict[str, torch.Tensor]:
    """Draw Q, K, V, dO on the CPU for ``case``.

    Returns CPU tensors already rounded to the case dtype (round-to-nearest-even
    through ``Tensor.to``).  ``B`` may shrink the batch for a bounded sample; the
    draw for batch index b does not depend on it only when B equals the case's
    batch, so a shrunken draw is a different (still seeded) sample.
    """
    b = case.B if B is None else B
    g = torch.Generator(device="cpu")
    g.manual_seed(case.seed)
    shapes = {
        "q": (b, case.Hq, case.Nq, case.d),
        "k": (b, case.Hkv, case.Nkv, case.d),
        "v": (b, case.Hkv, case.Nkv, case.d),
        "do": (b, case.Hq, case.Nq, case.d),
    }
    out = {}
    for key in ("q", "k", "v", "do"):
        if case.dist == "uniform":
            x = torch.rand(shapes[key], generator=g, dtype=torch.float32)
        else:
            x = torch.randn(shapes[key], generator=g, dtype=torch.float32)
        if key in ("q", "k") and case.qk_mult != 1.0:
            x = x * case.qk_mult
        out[key] = x.to(case.torch_dtype)
    return out


def make_custom(seed: int, B: int, Hq: int, Hkv: int, Nq: int, Nkv: int, d: int,
                dtype: str, dist: str = "normal", qk_mult: float = 1.0
                ) -> Dict[str, torch.Tensor]:
    """Seeded draw for an ad-hoc shape (edge-case tests)."""
    c = Case("custom", 0, seed, B, Hq, Hkv, Nq, Nkv, d, dtype, False, 1.0,
             dist=dist, qk_mult=qk_mult)
    return make_inputs(c)
