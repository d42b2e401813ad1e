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


# --- Additive bias and dropout --------------------------------------------------

EXT_FD_SHAPES = [
    # B, Hq, Hkv, Nq, Nkv, d, causal, bias shape, dropout p
    (1, 2, 1, 3, 6, 4, True, (1, 2, 3, 6), 0.3),
    (1, 2, 1, 4, 4, 4, False, (1, 1, 4, 4), 0.0),     # bias shared by the heads
    (1, 4, 2, 3, 5, 3, True, (1, 4, 1, 5), 0.5),     # per-key bias (a padding mask shape)
    (1, 1, 1, 5, 3, 2, True, (1, 1, 5, 3), 0.25),    # rows 0 and 1 see no key
]


def pin_ext_finite_differences(orc, seed=23) -> float:
    """Central differences of L = <dO, O(Q, K, V, bias)> with an additive bias and
    dropout (a fixed keep mask from the seed) against the oracle backward, bias
    gradient included (summed over the dimensions the bias is broadcast along)."""
    worst = 0.0
    rng = np.random.default_rng(seed)
    h = 1e-5
    for n, (B, Hq, Hkv, Nq, Nkv, d, causal, bshape, pdrop) in enumerate(EXT_FD_SHAPES):
        q = _rand(rng, (B, Hq, Nq, d))
        k = _rand(rng, (B, Hkv, Nkv, d))
        v = _rand(rng, (B, Hkv, Nkv, d))
        do = _rand(rng, (B, Hq, Nq, d))
        bias = _rand(rng, bshape)
        scale, rseed = 0.6, 1000 + n

        def loss(args):
            o, _ = orc.forward(args["q"], args["k"], args["v"], scale, causal, bias=args["bias"],
                               dropout_p=pdrop, seed=rseed)
            return float((o * do).sum())

        dq, dk, dv, dbias = orc.backward(q, k, v, do, scale, causal, bias=bias, dropout_p=pdrop,
                                         seed=rseed, return_dbias=True)
        # the gradient of a broadcast bias sums over the broadcast dimensions
        axes = tuple(i for i, (a, b_) in enumerate(zip(bshape, dbias.shape)) if a == 1 and b_ != 1)
        dbias_b = dbias.sum(axis=axes, keepdims=True)
        base = {"q": q, "k": k, "v": v, "bias": bias}
        for name, g in (("q", dq), ("k", dk), ("v", dv), ("bias", dbias_b)):
            x = base[name]
            fd = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                ap = dict(base); ap[name] = x.copy(); ap[name][idx] += h
                am = dict(base); am[name] = x.copy(); am[name][idx] -= h
                fd[idx] = (loss(ap) - loss(am)) / (2 * h)
            den = max(float(np.abs(fd).max()), 1.0)
            worst = max(worst, float(np.abs(fd - g).max()) / den)
    return worst


def pin_ext_row_variants(orc, seed=31) -> float:
    """Row-sampled functions with a bias and dropout against the whole-tensor ones
    (the mask of each element depends on its true batch, head, row and key), and
    dK/dV summed head by head (``heads=``) against the whole group."""
    worst = 0.0
    rng = np.random.default_rng(seed)
    for (B, Hq, Hkv, Nq, Nkv, d, causal, bshape, pdrop) in (
            (2, 4, 2, 13, 17, 8, True, (2, 1, 1, 17), 0.3),
            (1, 2, 1, 9, 9, 8, False, (1, 2, 9, 9), 0.5),
            (2, 2, 2, 11, 7, 4, True, None, 0.25)):
        q = _rand(rng, (B, Hq, Nq, d))
        k = _rand(rng, (B, Hkv, Nkv, d))
        v = _rand(rng, (B, Hkv, Nkv, d))
        do = _rand(rng, (B, Hq, Nq, d))
        bias = None if bshape is None else _rand(rng, bshape)
        kw = {"bias": bias, "dropout_p": pdrop, "seed": 4321}
        o, lse = orc.forward(q, k, v, 0.3, causal, **kw)
        dq, dk, dv = orc.backward(q, k, v, do, 0.3, causal, **kw)
        rows = np.array([0, 3, Nq - 2, Nq - 1])
        kv_rows = np.array([0, 1, Nkv - 2, Nkv - 1])
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                orow, lrow = orc.forward_rows(q, k, v, 0.3, causal, b, h, rows, **kw)
                fin = np.isfinite(lse[b, h, rows])
                worst = max(worst, _rel(orow, o[b, h, rows]),
                            float(np.abs(lrow[fin] - lse[b, h, rows][fin]).max(initial=0.0)))
                worst = max(worst, _rel(orc.dq_rows(q, k, v, do, 0.3, causal, b, h, rows, **kw),
                                        dq[b, h, rows]))
            for g in range(Hkv):
                dkr, dvr = orc.dkdv_rows(q, k, v, do, 0.3, causal, b, g, kv_rows, **kw)
                worst = max(worst, _rel(dkr, dk[b, g, kv_rows]), _rel(dvr, dv[b, g, kv_rows]))
                parts = [orc.dkdv_rows(q, k, v, do, 0.3, causal, b, g, kv_rows, heads=[h], **kw)
                         for h in range(g * G, (g + 1) * G)]
                worst = max(worst, _rel(sum(pp[0] for pp in parts), dkr),
                            _rel(sum(pp[1] for pp in parts), dvr))
    return worst


def pin_ext_identities(orc, seed=29) -> float:
    """With a bias and dropout: rowsum dS = 0, <Q,dQ> = <K,dK> (Q -> aQ, K -> K/a
    leaves the scores unchanged), <dO,O> = <V,dV> (L is linear in V); a zero bias
    and p = 0 reproduce the plain attention exactly; a bias constant along each
    row leaves O unchanged and shifts LSE by that constant; a bias of -inf on a
    set of keys is the attention over the remaining keys."""
    worst = 0.0
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Nq, Nkv, d = 1, 4, 2, 9, 11, 8
    q = _rand(rng, (B, Hq, Nq, d))
    k = _rand(rng, (B, Hkv, Nkv, d))
    v = _rand(rng, (B, Hkv, Nkv, d))
    do = _rand(rng, (B, Hq, Nq, d))
    bias = _rand(rng, (B, Hq, Nq, Nkv))
    for causal in (False, True):
        o, _ = orc.forward(q, k, v, 0.4, causal, bias=bias, dropout_p=0.4, seed=77)
        dq, dk, dv, ds = orc.backward(q, k, v, do, 0.4, causal, bias=bias, dropout_p=0.4, seed=77,
                                      return_dbias=True)
        worst = max(worst, float(np.abs(ds.sum(axis=-1)).max()) / float(np.abs(ds).max()))
        G = Hq // Hkv
        for g in range(Hkv):
            heads = range(g * G, (g + 1) * G)
            lhs = sum(float((q[0, h] * dq[0, h]).sum()) for h in heads)
            rhs = float((k[0, g] * dk[0, g]).sum())
            worst = max(worst, abs(lhs - rhs) / max(abs(rhs), 1e-300))
            lhs = sum(float((do[0, h] * o[0, h]).sum()) for h in heads)
            rhs = float((v[0, g] * dv[0, g]).sum())
            worst = max(worst, abs(lhs - rhs) / max(abs(rhs), 1e-300))
        plain = orc.forward(q, k, v, 0.4, causal)
        zero = orc.forward(q, k, v, 0.4, causal, bias=np.zeros((1, 1, 1, Nkv)), dropout_p=0.0)
        worst = max(worst, float(np.abs(plain[0] - zero[0]).max()))
        gp = orc.backward(q, k, v, do, 0.4, causal)
        gz = orc.backward(q, k, v, do, 0.4, causal, bias=np.zeros((1, 1, 1, Nkv)), dropout_p=0.0)
        worst = max(worst, max(float(np.abs(a - b_).max()) for a, b_ in zip(gp, gz)))
        shift = _rand(rng, (B, Hq, Nq, 1))
        o_s, l_s = orc.forward(q, k, v, 0.4, causal, bias=shift)
        fin = np.isfinite(plain[1])
        worst = max(worst, _rel(o_s, plain[0]), float(np.abs((l_s - plain[1])[fin] - shift[..., 0][fin]).max()))
    # -inf bias on keys 2, 5, 6 (non-causal) = attention over the other keys
    drop = [2, 5, 6]
    keep = [j for j in range(Nkv) if j not in drop]
    mb = np.zeros((1, 1, 1, Nkv)); mb[..., drop] = -np.inf
    o_m, l_m = orc.forward(q, k, v, 0.4, False, bias=mb)
    o_r, l_r = orc.forward(q, k[:, :, keep], v[:, :, keep], 0.4, False)
    worst = max(worst, _rel(o_m, o_r), float(np.abs(l_m - l_r).max()))
    gm = orc.backward(q, k, v, do, 0.4, False, bias=mb)
    gr = orc.backward(q, k[:, :, keep], v[:, :, keep], do, 0.4, False)
    worst = max(worst, _rel(gm[0], gr[0]), _rel(gm[1][:, :, keep], gr[1]), _rel(gm[2][:, :, keep], gr[2]))
    worst = max(worst, float(np.abs(gm[1][:, :, drop]).max()), float(np.abs(gm[2][:, :, drop]).max()))
    return worst


# Known-answer vectors of Philox4x32-10 published with the algorithm (the Random123
# library's test vectors by its authors): (counter, key) -> output words.
PHILOX4X32_KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def pin_philox(orc) -> float:
    """The generator: Philox4x32-10 against its published known-answer vectors;
    the same code at 64-bit words (Philox4x64-10) against NumPy's Philox bit
    generator, which increments its 256-bit counter before each block of four
    words; the dropout keep decisions against a per-element brute force of the
    definition; the keep rate against T / 256."""
    worst = 0.0
    for ctr, key, want in PHILOX4X32_KAT:
        got = orc.philox4(np.array([ctr], dtype=np.uint64), key)[0]
        worst = max(worst, float(sum(int(a) != b for a, b in zip(got, want))))
    gen = np.random.Philox(counter=[5, 0, 0, 0], key=[123456789, 987654321])
    raw = gen.random_raw(12).reshape(3, 4)
    for blk in range(3):
        got = orc.philox4(np.array([[6 + blk, 0, 0, 0]], dtype=np.uint64),
                          (123456789, 987654321), bits=64)[0]
        worst = max(worst, float(sum(int(a) != int(b) for a, b in zip(got, raw[blk]))))
    # brute force of the keep rule on a few (b, h, i, j)
    p, seed = 0.3, (7 << 32) | 12345
    t = orc.dropout_threshold(p)
    rows = np.arange(5, 14)
    z = orc.dropout_factors(1, 3, rows, 10, p, seed)
    for a, i in enumerate(rows):
        for j in range(10):
            w = orc.philox4(np.array([[j // 4, i // 4, 3, 1]], dtype=np.uint64),
                            (seed & 0xFFFFFFFF, seed >> 32))[0][i % 4]
            byte = (int(w) >> (8 * (j % 4))) & 0xFF
            want = 256.0 / t if byte < t else 0.0
            worst = max(worst, abs(z[a, j] - want))
    # threshold rule and extremes
    worst = max(worst, float(orc.dropout_threshold(0.0) != 256), float(orc.dropout_threshold(1.0) != 0),
                float(orc.dropout_threshold(0.5) != 128), float(orc.dropout_threshold(0.1) != 230),
                float(orc.dropout_threshold(0.7) != 77))  # 76.8 rounds up
    worst = max(worst, float(np.abs(orc.dropout_factors(0, 0, rows, 10, 0.0, seed) - 1.0).max()))
    worst = max(worst, float(np.abs(orc.dropout_factors(0, 0, rows, 10, 1.0, seed)).max()))
    # keep rate over 512 x 512 positions: within 6 standard deviations of T / 256
    z = orc.dropout_factors(2, 5, np.arange(512), 512, 0.2, 99)
    t = orc.dropout_threshold(0.2)
    rate, want = float((z > 0).mean()), t / 256.0
    sd = math.sqrt(want * (1 - want) / z.size)
    worst = max(worst, max(0.0, abs(rate - want) - 6 * sd))
    return worst


def pin_dropout_unbiased(orc) -> float:
    """Averaged over seeds, O with dropout is O without (each weight P_ij Z_ij has
    mean P_ij); the bound allows 6 standard errors of the mean of 400 draws."""
    rng = np.random.default_rng(31)
    q = _rand(rng, (1, 1, 3, 4))
    k = _rand(rng, (1, 1, 5, 4))
    v = _rand(rng, (1, 1, 5, 4))
    o_ref, _ = orc.forward(q, k, v, 0.5, False)
    draws = np.stack([orc.forward(q, k, v, 0.5, False, dropout_p=0.5, seed=s)[0] for s in range(400)])
    mean, sem = draws.mean(axis=0), draws.std(axis=0) / math.sqrt(draws.shape[0])
    return float(np.max(np.maximum(0.0, np.abs(mean - o_ref) - 6 * sem)))


ALL_PINS = [
    ("finite_differences", pin_finite_differences, FD_TOL),
    ("identities", pin_identities, IDENTITY_TOL),
    ("closed_forms", pin_closed_forms, CLOSED_TOL),
    ("naive_forward", pin_naive_forward, NAIVE_TOL),
    ("golden", pin_golden, GOLDEN_TOL),
    ("row_variants", pin_row_variants, NAIVE_TOL),
    ("ext_finite_differences", pin_ext_finite_differences, FD_TOL),
    ("ext_identities", pin_ext_identities, IDENTITY_TOL),
    ("ext_row_variants", pin_ext_row_variants, NAIVE_TOL),
    ("philox", pin_philox, 0.0),
    ("dropout_unbiased", pin_dropout_unbiased, 0.0),
]
