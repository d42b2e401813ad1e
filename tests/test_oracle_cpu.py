"""The fp64 oracle against mathematics: finite differences, gradient identities,
closed forms, an independent naive forward and hand-derived golden cases."""
import numpy as np
import pytest

import oracle.attention_fp64 as orc
from tests import oracle_pins as pins


@pytest.mark.parametrize("name,fn,tol", pins.ALL_PINS, ids=[p[0] for p in pins.ALL_PINS])
def test_pin(name, fn, tol):
    err = fn(orc)
    assert err <= tol, f"{name}: worst error {err:.3e} > {tol:.1e}"


def test_empty_rows_are_zero():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 6, 4))
    k = rng.standard_normal((1, 1, 3, 4))
    v = rng.standard_normal((1, 1, 3, 4))
    do = rng.standard_normal((1, 2, 6, 4))
    o, lse = orc.forward(q, k, v, 0.5, True)
    dq, dk, dv = orc.backward(q, k, v, do, 0.5, True)
    # N_q - N_kv = 3 top rows see no key
    assert np.all(lse[:, :, :3] == -np.inf)
    assert np.all(o[:, :, :3] == 0) and np.all(dq[:, :, :3] == 0)
    assert np.all(np.isfinite(lse[:, :, 3:]))


def test_zero_length_keys():
    q = np.ones((1, 1, 3, 4))
    k = np.zeros((1, 1, 0, 4))
    o, lse = orc.forward(q, k, k, 1.0, False)
    dq, dk, dv = orc.backward(q, k, k, q, 1.0, False)
    assert np.all(o == 0) and np.all(lse == -np.inf) and np.all(dq == 0)
    assert dk.shape == (1, 1, 0, 4)


def test_rounded_inputs_upcast_exactly():
    import torch
    from exact_attention_backward_fa_amd import inputs
    c = inputs.case_by_name("ragged_17x17_c")
    x = inputs.make_inputs(c)
    q64 = orc.as_f64(x["q"])
    assert q64.dtype == np.float64
    assert np.array_equal(q64, x["q"].double().numpy())
    assert x["q"].dtype == torch.float16


def test_inputs_are_seeded_and_shaped():
    from exact_attention_backward_fa_amd import inputs
    for c in inputs.cases_of_family(2):
        a, b = inputs.make_inputs(c), inputs.make_inputs(c)
        assert a["q"].shape == (c.B, c.Hq, c.Nq, c.d)
        assert a["k"].shape == (c.B, c.Hkv, c.Nkv, c.d)
        assert all(bool((a[t] == b[t]).all()) for t in a)
    seeds = [c.seed for c in inputs.all_cases()]
    assert len(seeds) == len(set(seeds)) == 1 + 8 + 1 + 20 + 2
    assert inputs.case_by_name("llama_gqa_bf16_8192").seed == 4000 + 2 * (13 - 5) + 1
    u = inputs.make_inputs(inputs.case_by_name("uniform"), B=1)
    assert float(u["q"].min()) >= 0.0 and float(u["q"].max()) <= 1.0
