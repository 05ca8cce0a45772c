"""Plain fp64 CPU oracle for the attention KL divergence KL(P1 || P2).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
nothing here imports the product package.

Pages cited (by title and section):
  [GS]  "StreamKL: Fast and Memory-Efficient KL Divergence for Boosting
        Attention Distillation", gist.science technical summary, sections
        "Problem Statement", "Methodology: StreamKL" (1 Online Formulation,
        2 Recomputation Strategy, 3 GPU Kernel Optimizations).
  [OA]  same title, OpenAlex record of the preprint (the authors' abstract).

What is computed, and from where:
  * P_t = softmax(S_t) row by row, S_t = scale * Q_t K_t^T, t = 1 (teacher),
    t = 2 (student); both are N_Q x N_K [GS, Problem Statement].
  * The per-row loss is the KL divergence of row i of P1 from row i of P2,
    KL_i = sum_j P1_ij * log(P1_ij / P2_ij) [GS, Problem Statement: an
    element-wise KL reduction over the two materialised distributions].  The
    oracle is exactly that definition: it materialises each row of P1 and P2
    (in log form, log P_t = S_t - LSE_t) and reduces it.  It does NOT use the
    streaming five-scalar recurrence of [GS, Methodology 1]; that recurrence is
    an exact rewrite of this sum and is what the GPU kernels implement.
  * LSE_t = log sum_j exp(S_t,ij) per row, in natural-log units
    [GS, Methodology 1: LSE_t = m_t + log l_t; Methodology 2: the saved state].
  * Backward [GS, Methodology 2 "Recomputation Strategy"]:
      Setting 1 - P1 held fixed, gradients flow to the student (Q2, K2);
      Setting 2 - P2 held fixed, gradients flow to the teacher (Q1, K1).
    With an upstream weight g_i per row (all ones when not given) the loss is
    sum_i g_i KL_i.  Its exact partial derivatives with respect to the logits
    (derived, the pages print none):
      Setting 1: dL/dS2_ij = g_i (P2_ij - P1_ij)                 (sum_j P1 = 1)
      Setting 2: dL/dS1_ij = g_i P1_ij (r_ij - KL_i),  r = log P1 - log P2
    where r is formed from logits and LSEs, not from log of probabilities
    [GS, Methodology 3 "Numerical Stability"].  Then
      dQ_t = scale * dS_t K_t   and   dK_t = scale * dS_t^T Q_t.
  * Causal masking [GS, Methodology 1: key tiles beyond the causal frontier are
    skipped]: the pages give no alignment for N_Q != N_K.  Reading adopted:
    bottom-right alignment, query i sees keys j <= i + (N_K - N_Q); causal with
    N_Q > N_K is not defined.  Masked pairs are simply absent from the row.

Reading of open points (the pages are silent): one caller-given softmax scale
for both distributions; natural logarithms; no reduction over rows (the forward
returns one KL value per row).

Every function here is pinned by tests/test_oracle_pins.py (brute force,
library autograd, finite differences, closed forms, invariants, the pages'
streaming identity).  No function is "parity unpinned".

Arithmetic: numpy fp64 throughout; the score matrix uses numpy's matmul as a
library primitive.  Rows are processed in blocks only to bound memory; each
row's computation is the plain definition above.
"""
from __future__ import annotations

import numpy as np

# Rows per block: bounds the materialised S block to ROW_BLOCK x N_K fp64.
ROW_BLOCK = 256


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def allowed_mask(rows: np.ndarray, n_q: int, n_k: int, causal: bool, keys=None) -> np.ndarray:
    """Boolean [len(rows), n_k] (or [len(rows), len(keys)] for a key subset):
    which keys query row i may attend to.

    Non-causal: every key.  Causal (bottom-right aligned): j <= i + (n_k - n_q).
    """
    rows = np.asarray(rows, dtype=np.int64)
    j = (np.arange(n_k, dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64))[None, :]
    if not causal:
        return np.ones((rows.size, j.shape[1]), dtype=bool)
    return j <= (rows[:, None] + (n_k - n_q))


def _log_softmax_rows(s: np.ndarray, mask: np.ndarray):
    """(log P, LSE) per row over the allowed keys; masked entries get -inf."""
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    lse = m + np.log(np.sum(np.exp(s - m), axis=1, keepdims=True))
    return s - lse, lse[:, 0]


def _row_block_state(q1, k1, q2, k2, scale, causal, rows):
    """Materialise rows of S1, S2, log P1, log P2 for one head."""
    n_q, n_k = q1.shape[0], k1.shape[0]
    mask = allowed_mask(rows, n_q, n_k, causal)
    s1 = scale * (q1[rows] @ k1.T)
    s2 = scale * (q2[rows] @ k2.T)
    lp1, lse1 = _log_softmax_rows(s1, mask)
    lp2, lse2 = _log_softmax_rows(s2, mask)
    return mask, lp1, lse1, lp2, lse2


def _kl_of_rows(mask, lp1, lp2):
    """KL_i = sum over allowed j of P1_ij * (log P1_ij - log P2_ij)."""
    p1 = np.exp(lp1)
    with np.errstate(invalid="ignore"):  # masked: 0 * (-inf - -inf), discarded
        terms = np.where(mask, p1 * (lp1 - lp2), 0.0)
    return np.sum(terms, axis=1)


def forward_head(q1, k1, q2, k2, scale: float, causal: bool, rows=None):
    """Per-row (KL, LSE1, LSE2) for one head.  Inputs are [N, d] arrays.

    rows: optional index array of query rows (default: all rows).
    Returns three fp64 arrays of len(rows).
    """
    q1, k1, q2, k2 = map(_as64, (q1, k1, q2, k2))
    n_q = q1.shape[0]
    if causal and n_q > k1.shape[0]:
        raise ValueError("causal attention needs n_q <= n_k")
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    kl = np.empty(rows.size)
    lse1 = np.empty(rows.size)
    lse2 = np.empty(rows.size)
    for b in range(0, rows.size, ROW_BLOCK):
        r = rows[b:b + ROW_BLOCK]
        mask, lp1, l1, lp2, l2 = _row_block_state(q1, k1, q2, k2, scale, causal, r)
        kl[b:b + r.size] = _kl_of_rows(mask, lp1, lp2)
        lse1[b:b + r.size] = l1
        lse2[b:b + r.size] = l2
    return kl, lse1, lse2


def _dlogits(setting: int, mask, lp1, lp2, kl, g):
    """dL/dS for the chosen setting, rows of one block (masked entries 0)."""
    p1 = np.exp(lp1)
    if setting == 1:
        ds = g[:, None] * (np.exp(lp2) - p1)
    elif setting == 2:
        with np.errstate(invalid="ignore"):  # masked: -inf - -inf, discarded
            r = np.where(mask, lp1 - lp2, 0.0)
        ds = g[:, None] * p1 * (r - kl[:, None])
    else:
        raise ValueError("setting must be 1 or 2")
    return np.where(mask, ds, 0.0)


def backward_head(setting: int, q1, k1, q2, k2, scale: float, causal: bool, dkl=None):
    """Full (dQ, dK) of sum_i g_i KL_i for one head.

    Setting 1 returns (dQ2, dK2); Setting 2 returns (dQ1, dK1).  fp64 [N, d].
    """
    q1, k1, q2, k2 = map(_as64, (q1, k1, q2, k2))
    n_q = q1.shape[0]
    g = np.ones(n_q) if dkl is None else _as64(dkl)
    q_t, k_t = (q2, k2) if setting == 1 else (q1, k1)
    dq = np.zeros_like(q_t)
    dk = np.zeros_like(k_t)
    for b in range(0, n_q, ROW_BLOCK):
        r = np.arange(b, min(n_q, b + ROW_BLOCK))
        mask, lp1, _, lp2, _ = _row_block_state(q1, k1, q2, k2, scale, causal, r)
        kl = _kl_of_rows(mask, lp1, lp2)
        ds = _dlogits(setting, mask, lp1, lp2, kl, g[r])
        dq[r] = scale * (ds @ k_t)
        dk += scale * (ds.T @ q_t[r])
    return dq, dk


def dlogits_head(setting: int, q1, k1, q2, k2, scale: float, causal: bool, dkl=None):
    """dL/dS of the chosen setting for one head, fp64 [N_Q, N_K] (masked entries 0)."""
    q1, k1, q2, k2 = map(_as64, (q1, k1, q2, k2))
    n_q = q1.shape[0]
    g = np.ones(n_q) if dkl is None else _as64(dkl)
    rows = np.arange(n_q)
    mask, lp1, _, lp2, _ = _row_block_state(q1, k1, q2, k2, scale, causal, rows)
    kl = _kl_of_rows(mask, lp1, lp2)
    return _dlogits(setting, mask, lp1, lp2, kl, g)


def dq_rows(setting: int, q1, k1, q2, k2, scale: float, causal: bool, rows, dkl=None):
    """dQ (of the chosen setting) for selected query rows only; exact per row."""
    q1, k1, q2, k2 = map(_as64, (q1, k1, q2, k2))
    rows = np.asarray(rows, dtype=np.int64)
    g_all = None if dkl is None else _as64(dkl)
    k_t = k2 if setting == 1 else k1
    out = np.empty((rows.size, q1.shape[1]))
    for b in range(0, rows.size, ROW_BLOCK):
        r = rows[b:b + ROW_BLOCK]
        mask, lp1, _, lp2, _ = _row_block_state(q1, k1, q2, k2, scale, causal, r)
        kl = _kl_of_rows(mask, lp1, lp2)
        g = np.ones(r.size) if g_all is None else g_all[r]
        ds = _dlogits(setting, mask, lp1, lp2, kl, g)
        out[b:b + r.size] = scale * (ds @ k_t)
    return out


def dk_keys(setting: int, q1, k1, q2, k2, scale: float, causal: bool, keys, dkl=None):
    """dK (of the chosen setting) for selected key rows; sums over all queries."""
    q1, k1, q2, k2 = map(_as64, (q1, k1, q2, k2))
    keys = np.asarray(keys, dtype=np.int64)
    n_q = q1.shape[0]
    g_all = np.ones(n_q) if dkl is None else _as64(dkl)
    q_t = q2 if setting == 1 else q1
    out = np.zeros((keys.size, q1.shape[1]))
    for b in range(0, n_q, ROW_BLOCK):
        r = np.arange(b, min(n_q, b + ROW_BLOCK))
        mask, lp1, _, lp2, _ = _row_block_state(q1, k1, q2, k2, scale, causal, r)
        kl = _kl_of_rows(mask, lp1, lp2)
        ds = _dlogits(setting, mask, lp1, lp2, kl, g_all[r])
        out += scale * (ds[:, keys].T @ q_t[r])
    return out


def dk_keys_from_state(setting: int, q1, k1, q2, k2, scale: float, causal: bool, keys,
                       lse1, lse2, kl, dkl=None):
    """dK (of the chosen setting) for selected key rows, given every query row's
    (LSE1, LSE2, KL) from forward_head.

    Same sum as dk_keys: dK_j = scale * sum_i dS_ij q_i, with dS_ij formed from
    the logits s_t,ij = scale q_t,i . k_t,j and the saved per-row statistics
    (log P_t,ij = s_t,ij - LSE_t,i), as the backward of the paper's Methodology
    ("Backward Pass": recomputation from the saved log-sum-exps) prescribes.
    Only the selected key columns are materialised, so the cost is
    O(N_Q * len(keys) * d) once the statistics exist.
    """
    q1, k1, q2, k2 = map(_as64, (q1, k1, q2, k2))
    lse1, lse2, kl = map(_as64, (lse1, lse2, kl))
    keys = np.asarray(keys, dtype=np.int64)
    n_q, n_k = q1.shape[0], k1.shape[0]
    g_all = np.ones(n_q) if dkl is None else _as64(dkl)
    q_t = q2 if setting == 1 else q1
    out = np.zeros((keys.size, q1.shape[1]))
    for b in range(0, n_q, ROW_BLOCK):
        r = np.arange(b, min(n_q, b + ROW_BLOCK))
        mask = allowed_mask(r, n_q, n_k, causal, keys)
        s1 = scale * (q1[r] @ k1[keys].T)
        s2 = scale * (q2[r] @ k2[keys].T)
        lp1 = np.where(mask, s1 - lse1[r, None], -np.inf)
        lp2 = np.where(mask, s2 - lse2[r, None], -np.inf)
        ds = _dlogits(setting, mask, lp1, lp2, kl[r], g_all[r])
        out += scale * (ds.T @ q_t[r])
    return out


# ---- multi-head conveniences: inputs [H, N, d] -------------------------------

def forward(q1, k1, q2, k2, scale: float, causal: bool):
    """(KL, LSE1, LSE2), each fp64 [H, N_Q], for all heads and rows."""
    outs = [forward_head(q1[h], k1[h], q2[h], k2[h], scale, causal) for h in range(q1.shape[0])]
    return tuple(np.stack([o[t] for o in outs]) for t in range(3))


def backward(setting: int, q1, k1, q2, k2, scale: float, causal: bool, dkl=None):
    """(dQ, dK) of the chosen setting, fp64 [H, N, d], for all heads."""
    outs = [backward_head(setting, q1[h], k1[h], q2[h], k2[h], scale, causal,
                          None if dkl is None else dkl[h]) for h in range(q1.shape[0])]
    return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
