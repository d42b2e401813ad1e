"""Checks that pin the fp64 oracle to mathematics rather than to itself.

Each ``pin_*`` function runs one family of checks against the oracle module it
is given and returns the worst error it saw (0.0 means exact agreement).
``tests/test_oracle_cpu.py`` asserts that every pin is below its bound;
``tests/test_oracle_mutants.py`` plants plausible mistakes in the oracle and
asserts that some pin then goes above its bound.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "closed_form.json")

# Bounds used by the CPU tests.
FD_TOL = 1e-6
IDENTITY_TOL = 1e-11
CLOSED_TOL = 1e-12
NAIVE_TOL = 1e-12
GOLDEN_TOL = 1e-12


def _rand(rng, shape, mult=1.0):
    return mult * rng.standard_normal(shape)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = max(float(np.max(np.abs(b))) if b.size else 0.0, 1e-300)
    return float(np.max(np.abs(a - b))) / den if a.size else 0.0


# Small shapes covering GQA, causal with N_q < N_kv, N_q = N_kv, N_q > N_kv
# (empty rows) and a single query row.
FD_SHAPES = [
    # B, Hq, Hkv, Nq, Nkv, d, causal
    (1, 2, 1, 1, 4, 4, False),
    (1, 2, 1, 3, 5, 4, True),
    (1, 2, 1, 3, 4, 4, False),
    (1, 2, 1, 1, 5, 4, True),
    (1, 4, 2, 3, 3, 3, True),
    (1, 1, 1, 5, 3, 2, True),   # rows 0 and 1 see no key
]


def pin_finite_differences(orc, seed=7) -> float:
    """Central differences of L = <dO, O(Q, K, V)> against the oracle backward."""
    worst = 0.0
    rng = np.random.default_rng(seed)
    h = 1e-5
    for (B, Hq, Hkv, Nq, Nkv, d, causal) in FD_SHAPES:
        q = _rand(rng, (B, Hq, Nq, d))
        k = _rand(rng, (B, Hkv, Nkv, d))
        v = _rand(rng, (B, Hkv, Nkv, d))
        do = _rand(rng, (B, Hq, Nq, d))
        scale = 0.7

        def loss(q_, k_, v_):
            o, _ = orc.forward(q_, k_, v_, scale, causal)
            return float((o * do).sum())

        dq, dk, dv = orc.backward(q, k, v, do, scale, causal)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}; args_p[name] = xp
                args_m = {"q": q, "k": k, "v": v}; args_m[name] = xm
                fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"])
                           - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            den = max(float(np.abs(fd).max()), 1.0)
            worst = max(worst, float(np.abs(fd - g).max()) / den)
    return worst


IDENTITY_SHAPES = [
    (2, 4, 2, 7, 9, 8, False),
    (1, 4, 2, 9, 9, 8, True),
    (1, 2, 2, 6, 11, 8, True),
    (1, 3, 1, 5, 5, 16, False),
]


def pin_identities(orc, seed=11) -> float:
    """rowsum dS = 0, sum_j dK_j = 0, sum_keys dV = sum_queries dO (no empty rows),
    <Q,dQ> = <K,dK> and <dO,O> = <V,dV> per key/value head."""
    worst = 0.0
    rng = np.random.default_rng(seed)
    for (B, Hq, Hkv, Nq, Nkv, d, causal) in IDENTITY_SHAPES:
        q = _rand(rng, (B, Hq, Nq, d))
        k = _rand(rng, (B, Hkv, Nkv, d))
        v = _rand(rng, (B, Hkv, Nkv, d))
        do = _rand(rng, (B, Hq, Nq, d))
        scale = 0.37
        o, _ = orc.forward(q, k, v, scale, causal)
        dq, dk, dv = orc.backward(q, k, v, do, scale, causal)
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                ds = orc.score_grad_matrix(q, k, v, do, scale, causal, b, h)
                worst = max(worst, float(np.abs(ds.sum(axis=1)).max())
                            / max(float(np.abs(ds).max()), 1e-300))
            for g in range(Hkv):
                heads = range(g * G, (g + 1) * G)
                scl = max(float(np.abs(dk[b, g]).max()), 1e-300)
                worst = max(worst, float(np.abs(dk[b, g].sum(axis=0)).max()) / scl)
                sum_do = sum(do[b, h].sum(axis=0) for h in heads)
                worst = max(worst, _rel(dv[b, g].sum(axis=0), sum_do))
                lhs = sum(float((q[b, h] * dq[b, h]).sum()) for h in heads)
                rhs = float((k[b, g] * dk[b, g]).sum())
                worst = max(worst, abs(lhs - rhs) / max(abs(rhs), 1e-300))
                lhs = sum(float((do[b, h] * o[b, h]).sum()) for h in heads)
                rhs = float((v[b, g] * dv[b, g]).sum())
                worst = max(worst, abs(lhs - rhs) / max(abs(rhs), 1e-300))
    return worst


def pin_closed_forms(orc, seed=13) -> float:
    """N_kv = 1 (non-causal): LSE = S_i0, O = V_0, dQ = dK = 0, dV = sum dO.
    Q = 0 (non-causal): LSE = ln N_kv, O = mean_j V_j."""
    worst = 0.0
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Nq, d, scale = 1, 4, 2, 6, 8, 0.5
    q = _rand(rng, (B, Hq, Nq, d))
    k = _rand(rng, (B, Hkv, 1, d))
    v = _rand(rng, (B, Hkv, 1, d))
    do = _rand(rng, (B, Hq, Nq, d))
    o, lse = orc.forward(q, k, v, scale, False)
    dq, dk, dv = orc.backward(q, k, v, do, scale, False)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        worst = max(worst, _rel(lse[0, h], scale * q[0, h] @ k[0, g, 0]))
        worst = max(worst, _rel(o[0, h], np.broadcast_to(v[0, g, 0], (Nq, d))))
    worst = max(worst, float(np.abs(dq).max()), float(np.abs(dk).max()))
    for g in range(Hkv):
        worst = max(worst, _rel(dv[0, g, 0], sum(do[0, h].sum(axis=0)
                                                 for h in range(g * G, (g + 1) * G))))
    Nkv = 7
    q0 = np.zeros((B, Hq, Nq, d))
    k = _rand(rng, (B, Hkv, Nkv, d))
    v = _rand(rng, (B, Hkv, Nkv, d))
    o, lse = orc.forward(q0, k, v, scale, False)
    worst = max(worst, float(np.abs(lse - math.log(Nkv)).max()))
    for h in range(Hq):
        worst = max(worst, _rel(o[0, h], np.broadcast_to(v[0, h // G].mean(axis=0), (Nq, d))))
    return worst


NAIVE_SHAPES = [
    (1, 4, 2, 5, 9, 8, True),
    (2, 2, 1, 9, 5, 8, True),     # N_q > N_kv: top rows empty
    (1, 3, 3, 6, 6, 4, False),
    (1, 4, 1, 1, 13, 8, True),
]


def pin_naive_forward(orc, seed=17) -> float:
    """The log-sum-exp forward against an independently written softmax forward,
    including a mask count check (causal N_q = N_kv keeps N(N+1)/2 entries)."""
    worst = 0.0
    rng = np.random.default_rng(seed)
    for (B, Hq, Hkv, Nq, Nkv, d, causal) in NAIVE_SHAPES:
        q = _rand(rng, (B, Hq, Nq, d), 1.5)
        k = _rand(rng, (B, Hkv, Nkv, d), 1.5)
        v = _rand(rng, (B, Hkv, Nkv, d))
        o, lse = orc.forward(q, k, v, 0.4, causal)
        on = orc.naive_forward(q, k, v, 0.4, causal)
        worst = max(worst, _rel(o, on))
        # LSE against a direct log of the sum of exp over visible keys
        for b in range(B):
            for h in range(Hq):
                for i in range(Nq):
                    vis = [j for j in range(Nkv) if not causal or j <= i + Nkv - Nq]
                    if vis:
                        ref = math.log(sum(math.exp(0.4 * float(q[b, h, i] @ k[b, h // (Hq // Hkv), j]))
                                           for j in vis))
                        worst = max(worst, abs(lse[b, h, i] - ref) / max(abs(ref), 1.0))
                    elif lse[b, h, i] != -np.inf:
                        worst = max(worst, 1.0)
    n = 11
    kept = int(orc.keep_mask(np.arange(n), n, n, True).sum())
    worst = max(worst, abs(kept - n * (n + 1) // 2))
    n_q, n_kv = 4, 10
    kept = orc.keep_mask(np.arange(n_q), n_q, n_kv, True).sum(axis=1)
    worst = max(worst, float(np.abs(kept - (np.arange(n_q) + n_kv - n_q + 1)).max()))
    return worst


def _golden_arr(x):
    return np.array(x, dtype=object).astype(np.float64)


def pin_golden(orc) -> float:
    """Hand-derived closed-form cases stored under tests/golden/."""
    worst = 0.0
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["cases"]:
        q, k, v, do = (_golden_arr(c[key]) for key in ("q", "k", "v", "do"))
        o, lse = orc.forward(q, k, v, c["scale"], c["causal"])
        dq, dk, dv = orc.backward(q, k, v, do, c["scale"], c["causal"])
        exp_lse = _golden_arr(c["lse"])
        fin = np.isfinite(exp_lse)
        if not np.array_equal(fin, np.isfinite(lse)):
            worst = max(worst, 1.0)
        else:
            worst = max(worst, float(np.abs(lse[fin] - exp_lse[fin]).max()) if fin.any() else 0.0)
        for got, key in ((o, "o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
            worst = max(worst, float(np.abs(got - _golden_arr(c[key])).max()))
    return worst


def pin_row_variants(orc, seed=19) -> float:
    """Row-sampled functions against the whole-tensor ones."""
    worst = 0.0
    rng = np.random.default_rng(seed)
    for (B, Hq, Hkv, Nq, Nkv, d, causal) in ((1, 4, 2, 13, 17, 8, True),
                                              (1, 2, 2, 9, 9, 8, False)):
        q = _rand(rng, (B, Hq, Nq, d))
        k = _rand(rng, (B, Hkv, Nkv, d))
        v = _rand(rng, (B, Hkv, Nkv, d))
        do = _rand(rng, (B, Hq, Nq, d))
        o, lse = orc.forward(q, k, v, 0.3, causal)
        dq, dk, dv = orc.backward(q, k, v, do, 0.3, causal)
        rows = np.array([0, 3, Nq - 1])
        for h in range(Hq):
            orow, lrow = orc.forward_rows(q, k, v, 0.3, causal, 0, h, rows)
            worst = max(worst, _rel(orow, o[0, h, rows]), float(np.abs(lrow - lse[0, h, rows]).max()))
            worst = max(worst, _rel(orc.dq_rows(q, k, v, do, 0.3, causal, 0, h, rows), dq[0, h, rows]))
        kv_rows = np.array([1, Nkv - 2, Nkv - 1])
        for g in range(Hkv):
            dkr, dvr = orc.dkdv_rows(q, k, v, do, 0.3, causal, 0, g, kv_rows)
            worst = max(worst, _rel(dkr, dk[0, g, kv_rows]), _rel(dvr, dv[0, g, kv_rows]))
    return worst


ALL_PINS = [
    ("finite_differences", pin_finite_differences, FD_TOL),
    ("identities", pin_identities, IDENTITY_TOL),
    ("closed_forms", pin_closed_forms, CLOSED_TOL),
    ("naive_forward", pin_naive_forward, NAIVE_TOL),
    ("golden", pin_golden, GOLDEN_TOL),
    ("row_variants", pin_row_variants, NAIVE_TOL),
]
