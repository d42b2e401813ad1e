"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: a dropped term, a wrong sign, a transposed operand, a missing
scale, a wrong mask alignment, a wrong GQA mapping, a wrong log base."""
import numpy as np
import pytest

import oracle.attention_fp64 as orc
from tests import oracle_pins as pins

MUTANTS = {
    "dS_drops_D": ("score_grad", lambda p, dp, dlt: p * dp),
    "dS_wrong_sign": ("score_grad", lambda p, dp, dlt: p * (dlt[:, None] - dp)),
    "dK_missing_scale": ("grad_k", lambda ds, q, scale: ds.T @ q),
    "dQ_missing_scale": ("grad_q", lambda ds, k, scale: ds @ k),
    "dV_uses_P_not_PT": ("grad_v", lambda p, do: (p @ do) if p.shape[0] == p.shape[1] else p.T @ (do * 0.5)),
    "dK_transposed_dS": ("grad_k", lambda ds, q, scale: scale * (ds @ q) if ds.shape[0] == ds.shape[1] else scale * ds.T @ q * 0.5),
    "mask_top_left": ("keep_mask", lambda rows, nq, nkv, causal:
                      (np.arange(nkv)[None, :] <= np.asarray(rows)[:, None]) if causal
                      else np.ones((len(rows), nkv), bool)),
    "gqa_modulo": ("kv_head_index", lambda h, hq, hkv: h % hkv),
    "lse_log2": ("log_sum_exp", lambda s: orc_lse_log2(s)),
    # additive bias and dropout
    "bias_subtracted": ("masked_scores", lambda q, k, scale, keep, bias=None:
                        _ORIG_SCORES(q, k, scale, keep, None if bias is None else -bias)),
    "dropout_not_rescaled": ("dropout_factors", lambda *a: np.minimum(_ORIG_DROP(*a), 1.0)),
    "dropout_keeps_above_threshold": ("dropout_factors", lambda *a: orc_drop_inverted(*a)),
    "philox_no_key_bump": ("philox4", lambda ctr, key, bits=32, rounds=10:
                           orc_philox_no_bump(ctr, key, bits, rounds)),
    "threshold_truncated": ("dropout_threshold", lambda p: int(np.floor((np.float32(1) - np.float32(p))
                                                                        * np.float32(256)))),
}

_ORIG_LSE = orc.log_sum_exp
_ORIG_SCORES = orc.masked_scores
_ORIG_DROP = orc.dropout_factors
_ORIG_PHILOX = orc.philox4


def orc_lse_log2(s):
    return _ORIG_LSE(s) / np.log(2.0)


def orc_drop_inverted(b, h, rows, n_keys, p, seed):
    """keep where the byte is at or above the threshold (the complement rule)"""
    z = _ORIG_DROP(b, h, rows, n_keys, p, seed)
    t = orc.dropout_threshold(p)
    if t in (0, 256):
        return z
    return np.where(z > 0, 0.0, 256.0 / (256 - t))


def orc_philox_no_bump(ctr, key, bits, rounds):
    """every round with the unbumped key"""
    out = np.asarray(ctr, dtype=np.uint64)
    for _ in range(rounds):
        out = _ORIG_PHILOX(out, key, bits, 1)
    return out


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for name, pin, tol in pins.ALL_PINS:
        try:
            err = pin(orc)
        except Exception:  # a mutant that breaks shapes is caught too
            err = float("inf")
        if not err <= tol:
            caught.append(name)
    assert caught, f"no pin catches mutant {mutant}"
