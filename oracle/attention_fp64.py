"""fp64 CPU oracle for exact softmax attention: forward (O, LSE) and backward
(dQ, dK, dV).

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports this module; only the
tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may call
it.  It shares no code with the HIP kernels and is deliberately slow: it
materialises the score matrix S, the probabilities P and the score gradient dS
(row chunks bound the memory), in float64, with NumPy's ``exp``/``log`` and
BLAS matrix products as the only library steps.

What is computed (the tiled method of the pages reaches exactly this gradient,
up to rounding order, because it only reorders the same sums):

* scores      S = scale * Q_h K_g^T, with masked entries set to -inf
  (rustytorch "flash_attention_backward.cu": the score recompute and causal mask
  step of the tiled backward kernel; Triton issue "Extra transposes cause 8x
  speedup ...": ``qk = q k^T * scale`` in ``_bwd_kernel``);
* LSE_i       = log sum_j exp(S_ij), natural log, in the scaled-score domain;
  P = exp(S - LSE) (the same two pages: probabilities rebuilt from the stored
  per-row log-sum-exp);
* O           = P V;
* D_i         = sum_d dO_id O_id (rustytorch page: the per-row dot product of dO
  and O; Triton page: the precomputed ``D`` loaded per query row);
* dP          = dO V^T;  dS = P o (dP - D)  (rustytorch page: the dS step;
  Triton page: ``ds = p * (dp - Di)``);
* dQ          = scale * dS K;  dK = sum_{h in g} scale * dS^T Q_h;
  dV          = sum_{h in g} P^T dO_h (rustytorch page: the dQ/dK/dV
  accumulation; Triton page: ``dv += p^T do``, ``dk += ds^T q``, ``dq = ds k``).

Readings where the pages are silent or disagree:

* Causal masking is bottom-right aligned: query i may see key j iff
  j <= i + (N_kv - N_q).  (The rustytorch kernel masks k_pos > q_pos with one
  shared length, which is the N_q = N_kv special case of this rule.)
* GQA maps query head h to key/value head h // (Hq/Hkv): consecutive query
  heads share a key/value head (the Liger-Kernel pull request "[Kernel] Flash
  attention 2" lists GQA without fixing the mapping).
* A query row with no visible key (causal with N_q > N_kv, or N_kv = 0) has
  O = 0, LSE = -inf and a zero dQ row; it contributes nothing to dK and dV.
* The rustytorch kernel sums dQ over every row of a tile into one vector and
  stores it to each row; that is a defect, and the oracle follows the
  definition dQ = scale * dS K row by row instead.
* The scale is applied to dS once, in the dQ and dK products; folding it into
  dS first (Triton page) is the same number.

Two optional extensions of the scores and probabilities (both off by default,
when the arithmetic above is exactly what runs):

* an additive bias: S = scale * Q_h K_g^T + bias_h (the Liger-Kernel pull
  request "[Kernel] Flash attention 2", Details, lists an attention mask and an
  attention bias); the bias is part of the score, so its gradient is the score
  gradient, dBias = dS;
* dropout of the probabilities: O = (P o Z) V with Z = keep / (1 - p) (the same
  page, Details: dropout in the forward, its gradient left unsolved there).  Then
  dV = (P o Z)^T dO, dP = (dO V^T) o Z, and D = rowsum(dO o O) and
  dS = P o (dP - D) keep their form.  The keep decisions come from the
  counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011), one call per 4 x 4 block of
  (query, key) positions: counter (key // 4, query // 4, query head, batch), key =
  the 64-bit seed's low and high words; element (i, j) keeps iff byte j % 4 of
  output word i % 4 is below T = floor((1 - p) * 256 + 1/2) (float32 arithmetic),
  so the keep probability is T / 256 and Z = 256 / T on kept elements.

Pinned (tests/test_oracle_cpu.py) by central finite differences of
L = <dO, O>, the identities sum_j dS_ij = 0, sum_j dK_j = 0,
sum_keys dV = sum_queries dO, <Q, dQ> = <K, dK>, <V, dV> = <dO, O>, closed forms
(N_kv = 1; Q = 0), an independently written naive softmax forward, pure-Python
brute force on a tiny case, and analytic golden fixtures.
"""
from __future__ import annotations

import numpy as np

# Rows of S handled at once; bounds the temporary S/P/dS blocks to
# ROW_CHUNK * N_kv float64 values each.
ROW_CHUNK = 1024


def as_f64(x) -> np.ndarray:
    """Exact upcast of a float16/bfloat16/float32 tensor or array to float64."""
    if hasattr(x, "detach"):  # torch tensor: go through float32, which is exact
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head_index(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head serving query head h: consecutive groups of Hq/Hkv."""
    return h // (Hq // Hkv)


def keep_mask(rows: np.ndarray, Nq: int, Nkv: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), Nkv]: True where query row i may attend key j.

    Causal is bottom-right aligned: keep iff j <= i + (Nkv - Nq).
    """
    rows = np.asarray(rows)
    if not causal:
        return np.ones((rows.shape[0], Nkv), dtype=bool)
    j = np.arange(Nkv)
    return j[None, :] <= rows[:, None] + (Nkv - Nq)


def masked_scores(q_rows: np.ndarray, k: np.ndarray, scale: float,
                  keep: np.ndarray, bias_rows=None) -> np.ndarray:
    """S = scale * q_rows k^T (+ bias_rows) with masked entries at -inf."""
    s = scale * (q_rows @ k.T)
    if bias_rows is not None:
        s = s + bias_rows
    return np.where(keep, s, -np.inf)


def log_sum_exp(s: np.ndarray) -> np.ndarray:
    """Per-row natural-log sum of exp(S); -inf for a row with every entry masked."""
    m = s.max(axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    with np.errstate(under="ignore"):
        tot = np.exp(s - m_safe[:, None]).sum(axis=1)
    out = m_safe + np.log(np.where(empty, 1.0, tot))
    return np.where(empty, -np.inf, out)


def probabilities(s: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """P = exp(S - LSE); zero on masked entries and on empty rows."""
    lse_safe = np.where(np.isfinite(lse), lse, np.inf)
    with np.errstate(under="ignore", invalid="ignore"):
        p = np.exp(s - lse_safe[:, None])
    return np.where(np.isfinite(s) & np.isfinite(lse)[:, None], p, 0.0)


def row_delta(do_rows: np.ndarray, o_rows: np.ndarray) -> np.ndarray:
    """D_i = sum_d dO_id * O_id."""
    return (do_rows * o_rows).sum(axis=1)


def score_grad(p: np.ndarray, dp: np.ndarray, dlt: np.ndarray) -> np.ndarray:
    """dS = P o (dP - D): gradient of the loss with respect to the scaled scores."""
    return p * (dp - dlt[:, None])


# --- Counter-based generator and dropout keep decisions ---------------------------

# Philox constants of the paper: round multipliers M and key increments W (the
# golden ratio and sqrt(3) - 1 in fixed point), per word width.
PHILOX = {
    32: ((0xD2511F53, 0xCD9E8D57), (0x9E3779B9, 0xBB67AE85)),
    64: ((0xD2E7470EE14C6C93, 0xCA5A826395121157), (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)),
}


def _mulhilo(m: int, x: np.ndarray, bits: int):
    """(high, low) words of the 2*bits-bit product m * x (x: uint64 array of words)."""
    if bits == 32:
        prod = x * np.uint64(m)
        return prod >> np.uint64(32), prod & np.uint64(0xFFFFFFFF)
    # 64-bit words: schoolbook product of 32-bit halves
    lo32 = np.uint64(0xFFFFFFFF)
    m1, m0 = np.uint64(m >> 32), np.uint64(m & 0xFFFFFFFF)
    x1, x0 = x >> np.uint64(32), x & lo32
    p00, p01, p10, p11 = x0 * m0, x0 * m1, x1 * m0, x1 * m1
    mid = (p00 >> np.uint64(32)) + (p01 & lo32) + (p10 & lo32)
    lo = (p00 & lo32) | ((mid & lo32) << np.uint64(32))
    hi = p11 + (p01 >> np.uint64(32)) + (p10 >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4(ctr, key, bits: int = 32, rounds: int = 10) -> np.ndarray:
    """Philox4xW-R: counter words ctr[..., 0..3], key words (k0, k1); returns the
    four output words [..., 4] as uint64 (each < 2^bits).  A round maps
    (c0, c1, c2, c3) to (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)); the key is bumped by W before every round but the first."""
    (m0, m1), (w0, w1) = PHILOX[bits]
    mask = (1 << bits) - 1
    ctr = np.asarray(ctr, dtype=np.uint64)
    c0, c1, c2, c3 = (ctr[..., i].copy() for i in range(4))
    k0, k1 = int(key[0]) & mask, int(key[1]) & mask
    for r in range(rounds):
        if r > 0:
            k0, k1 = (k0 + w0) & mask, (k1 + w1) & mask
        hi0, lo0 = _mulhilo(m0, c0, bits)
        hi1, lo1 = _mulhilo(m1, c2, bits)
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return np.stack([c0, c1, c2, c3], axis=-1)


def dropout_threshold(p: float) -> int:
    """T = floor((1 - p) * 256 + 1/2) in float32 arithmetic, clamped to [0, 256]:
    an element is kept iff its random byte is below T."""
    one, p32 = np.float32(1.0), np.float32(p)
    t = np.floor((one - p32) * np.float32(256.0) + np.float32(0.5))
    return int(min(max(t, 0.0), 256.0))


def dropout_factors(b: int, h: int, rows, n_keys: int, p: float, seed: int) -> np.ndarray:
    """Z [len(rows), n_keys]: 256 / T where (query row, key) is kept, else 0."""
    rows = np.asarray(rows, dtype=np.int64)
    t = dropout_threshold(p)
    if t >= 256:
        return np.ones((rows.shape[0], n_keys))
    if t == 0:
        return np.zeros((rows.shape[0], n_keys))
    kb = np.arange((n_keys + 3) // 4, dtype=np.uint64)
    ctr = np.zeros((rows.shape[0], kb.shape[0], 4), dtype=np.uint64)
    ctr[..., 0] = kb[None, :]
    ctr[..., 1] = (rows >> 2).astype(np.uint64)[:, None]
    ctr[..., 2] = h
    ctr[..., 3] = b
    words = philox4(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))  # [R, Kb, 4]
    j = np.arange(n_keys)
    w = words[:, j >> 2, :]                                                 # [R, n_keys, 4]
    word = np.take_along_axis(w, (rows & 3)[:, None, None], axis=2)[..., 0]
    byte = (word >> (np.uint64(8) * (j & 3).astype(np.uint64))[None, :]) & np.uint64(0xFF)
    return np.where(byte < np.uint64(t), 256.0 / t, 0.0)


def grad_q(ds: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    return scale * (ds @ k)


def grad_k(ds: np.ndarray, q_rows: np.ndarray, scale: float) -> np.ndarray:
    return scale * (ds.T @ q_rows)


def grad_v(p: np.ndarray, do_rows: np.ndarray) -> np.ndarray:
    return p.T @ do_rows


def _check_shapes(q, k, v):
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nkv, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d or Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"bad shapes q={q.shape} k={k.shape} v={v.shape}")
    return B, Hq, Hkv, Nq, Nkv, d


def _row_chunks(rows: np.ndarray):
    for s in range(0, rows.shape[0], ROW_CHUNK):
        yield rows[s:s + ROW_CHUNK]


def _bias_of(bias, B, Hq, Nq, Nkv):
    """The bias broadcast to [B, Hq, Nq, Nkv] in float64 (None stays None)."""
    if bias is None:
        return None
    return np.broadcast_to(as_f64(bias), (B, Hq, Nq, Nkv))


def _dropout_of(b, h, rows, Nkv, dropout_p, seed):
    if dropout_p == 0.0:
        return None
    return dropout_factors(b, h, rows, Nkv, dropout_p, seed)


def forward(q, k, v, scale: float, causal: bool, bias=None, dropout_p: float = 0.0,
            seed: int = 0):
    """O [B,Hq,Nq,d] and LSE [B,Hq,Nq] in float64.  ``bias``: broadcastable to
    [B,Hq,Nq,Nkv], added to the scores; ``dropout_p``, ``seed``: dropout of P."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Hq, Hkv, Nq, Nkv, d = _check_shapes(q, k, v)
    bias = _bias_of(bias, B, Hq, Nq, Nkv)
    o = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_index(h, Hq, Hkv)
            for rows in _row_chunks(np.arange(Nq)):
                s = masked_scores(q[b, h, rows], k[b, g], scale,
                                  keep_mask(rows, Nq, Nkv, causal),
                                  None if bias is None else bias[b, h, rows])
                l_ = log_sum_exp(s)
                p = probabilities(s, l_)
                z = _dropout_of(b, h, rows, Nkv, dropout_p, seed)
                o[b, h, rows] = (p if z is None else p * z) @ v[b, g]
                lse[b, h, rows] = l_
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool, return_delta: bool = False,
             bias=None, dropout_p: float = 0.0, seed: int = 0, return_dbias: bool = False):
    """dQ, dK, dV in float64 from the definition (O and LSE recomputed here).

    With ``return_delta`` also returns D [B,Hq,Nq] computed from the oracle's
    own float64 O; with ``return_dbias`` also dBias = dS [B,Hq,Nq,Nkv] (last).
    ``bias``, ``dropout_p`` and ``seed`` as in ``forward``.
    """
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, Hq, Hkv, Nq, Nkv, d = _check_shapes(q, k, v)
    bias = _bias_of(bias, B, Hq, Nq, Nkv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dlt_all = np.zeros((B, Hq, Nq))
    dbias = np.zeros((B, Hq, Nq, Nkv)) if return_dbias else None
    for b in range(B):
        for h in range(Hq):
            g = kv_head_index(h, Hq, Hkv)
            for rows in _row_chunks(np.arange(Nq)):
                qr, dor = q[b, h, rows], do[b, h, rows]
                s = masked_scores(qr, k[b, g], scale, keep_mask(rows, Nq, Nkv, causal),
                                  None if bias is None else bias[b, h, rows])
                p = probabilities(s, log_sum_exp(s))
                z = _dropout_of(b, h, rows, Nkv, dropout_p, seed)
                pz = p if z is None else p * z          # the probabilities V is weighted by
                o_rows = pz @ v[b, g]
                dlt = row_delta(dor, o_rows)
                dp = dor @ v[b, g].T
                if z is not None:
                    dp = dp * z
                ds = score_grad(p, dp, dlt)
                dq[b, h, rows] = grad_q(ds, k[b, g], scale)
                dk[b, g] += grad_k(ds, qr, scale)
                dv[b, g] += grad_v(pz, dor)
                dlt_all[b, h, rows] = dlt
                if dbias is not None:
                    dbias[b, h, rows] = ds
    out = (dq, dk, dv)
    if return_delta:
        out = out + (dlt_all,)
    if return_dbias:
        out = out + (dbias,)
    return out


def score_grad_matrix(q, k, v, do, scale: float, causal: bool, b: int, h: int):
    """The full dS matrix of one (batch, query head); for identity checks."""
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, Hq, Hkv, Nq, Nkv, d = _check_shapes(q, k, v)
    g = kv_head_index(h, Hq, Hkv)
    rows = np.arange(Nq)
    s = masked_scores(q[b, h], k[b, g], scale, keep_mask(rows, Nq, Nkv, causal))
    p = probabilities(s, log_sum_exp(s))
    dlt = row_delta(do[b, h], p @ v[b, g])
    return score_grad(p, do[b, h] @ v[b, g].T, dlt)


def naive_forward(q, k, v, scale: float, causal: bool):
    """softmax(scale * Q K^T) V written without a log-sum-exp: normalise
    exp(S - rowmax) by its row sum.  Written separately from ``forward`` so the
    two can be compared; O only."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Hq, Hkv, Nq, Nkv, d = _check_shapes(q, k, v)
    out = np.zeros((B, Hq, Nq, d))
    for b in range(B):
        for h in range(Hq):
            kk = k[b, h // (Hq // Hkv)]
            vv = v[b, h // (Hq // Hkv)]
            for i in range(Nq):
                allowed = [j for j in range(Nkv) if (not causal) or j - i <= Nkv - Nq]
                if not allowed:
                    continue
                logits = np.array([scale * float(np.dot(q[b, h, i], kk[j])) for j in allowed])
                w = np.exp(logits - logits.max())
                w = w / w.sum()
                out[b, h, i] = w @ vv[allowed]
    return out


# --- Row-sampled variants for shapes too large to materialise whole --------------

def forward_rows(q, k, v, scale: float, causal: bool, b: int, h: int, rows, bias=None,
                 dropout_p: float = 0.0, seed: int = 0):
    """O and LSE of selected query rows of one (batch, head); cost O(len(rows)*Nkv*d).
    ``bias``, ``dropout_p`` and ``seed`` as in ``forward``."""
    rows = np.asarray(rows)
    B, Hq, Nq = q.shape[0], q.shape[1], q.shape[2]
    Hkv, Nkv = k.shape[1], k.shape[2]
    g = kv_head_index(h, Hq, Hkv)
    bias = _bias_of(bias, B, Hq, Nq, Nkv)
    qr = as_f64(q[b, h][rows])
    kg, vg = as_f64(k[b, g]), as_f64(v[b, g])
    s = masked_scores(qr, kg, scale, keep_mask(rows, Nq, Nkv, causal),
                      None if bias is None else bias[b, h, rows])
    l_ = log_sum_exp(s)
    p = probabilities(s, l_)
    z = _dropout_of(b, h, rows, Nkv, dropout_p, seed)
    return (p if z is None else p * z) @ vg, l_


def dq_rows(q, k, v, do, scale: float, causal: bool, b: int, h: int, rows, bias=None,
            dropout_p: float = 0.0, seed: int = 0):
    """dQ of selected query rows; each row needs only its own S, P and dP rows.
    ``bias``, ``dropout_p`` and ``seed`` as in ``forward``."""
    rows = np.asarray(rows)
    B, Hq, Nq = q.shape[0], q.shape[1], q.shape[2]
    Hkv, Nkv = k.shape[1], k.shape[2]
    g = kv_head_index(h, Hq, Hkv)
    bias = _bias_of(bias, B, Hq, Nq, Nkv)
    qr, dor = as_f64(q[b, h][rows]), as_f64(do[b, h][rows])
    kg, vg = as_f64(k[b, g]), as_f64(v[b, g])
    s = masked_scores(qr, kg, scale, keep_mask(rows, Nq, Nkv, causal),
                      None if bias is None else bias[b, h, rows])
    p = probabilities(s, log_sum_exp(s))
    z = _dropout_of(b, h, rows, Nkv, dropout_p, seed)
    dp = dor @ vg.T
    if z is not None:
        dp = dp * z
    ds = score_grad(p, dp, row_delta(dor, (p if z is None else p * z) @ vg))
    return grad_q(ds, kg, scale)


def dkdv_rows(q, k, v, do, scale: float, causal: bool, b: int, g: int, kv_rows, bias=None,
              dropout_p: float = 0.0, seed: int = 0, heads=None):
    """dK and dV of selected key rows of one (batch, kv head).

    Only query rows that can see one of the selected keys contribute; with a
    causal mask and keys near the end of the sequence that is a short tail, so
    this stays cheap at any length.  ``heads``: the query heads of the group to
    sum over (default all of them).  ``bias``, ``dropout_p`` and ``seed`` as in
    ``forward``.
    """
    kv_rows = np.asarray(kv_rows)
    B, Hq, Nq, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    bias = _bias_of(bias, B, Hq, Nq, Nkv)
    kg, vg = as_f64(k[b, g]), as_f64(v[b, g])
    dk_out = np.zeros((kv_rows.shape[0], d))
    dv_out = np.zeros((kv_rows.shape[0], d))
    first = 0
    if causal and kv_rows.shape[0] > 0:
        first = max(0, int(kv_rows.min()) - (Nkv - Nq))
    contributing = np.arange(first, Nq)
    for h in range(Hq) if heads is None else heads:
        if kv_head_index(h, Hq, Hkv) != g:
            continue
        for rows in _row_chunks(contributing):
            qr, dor = as_f64(q[b, h][rows]), as_f64(do[b, h][rows])
            # LSE and D need whole rows of S and P; dP and dS only the selected
            # key columns
            s = masked_scores(qr, kg, scale, keep_mask(rows, Nq, Nkv, causal),
                              None if bias is None else bias[b, h, rows])
            p = probabilities(s, log_sum_exp(s))
            z = _dropout_of(b, h, rows, Nkv, dropout_p, seed)
            pz = p if z is None else p * z
            dlt = row_delta(dor, pz @ vg)
            dp_sel = dor @ vg[kv_rows].T
            if z is not None:
                dp_sel = dp_sel * z[:, kv_rows]
            ds_sel = score_grad(p[:, kv_rows], dp_sel, dlt)
            dk_out += grad_k(ds_sel, qr, scale)
            dv_out += grad_v(pz[:, kv_rows], dor)
    return dk_out, dv_out
