"""Plain, slow fp64 CPU oracle for the attention KL divergence KL(P1 || P2).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the GPU library and never calls it.

What it computes is the plain definition, materialised one block of query rows
at a time (never the streaming recurrence):

* "StreamKL" technical summary (gist.science, ja/fr/ko), Problem statement:
  the two attention distributions P1, P2 in R^{N_Q x N_K}, each a row-wise
  softmax of scaled query-key logits, and the row-wise KL reduction over them.
* Same page, Method 1 (online formulation): the objective per row is
  L = acc/l1 + LSE2 - LSE1 with LSE_t = m_t + log l_t.  That identity holds
  exactly for KL(P1 || P2) with the expectation taken under P1, so the KL
  direction is P1 (teacher, "fixed" in setting 1) against P2.
* Same page, Method 2 (recomputation strategy): the stored state is the KL row
  values and LSE1, LSE2; probabilities are P_t = exp(S_t - LSE_t); setting 1
  keeps P1 fixed and trains P2, setting 2 keeps P2 fixed and trains P1.
* Same page, Method 3 (numerical stability): the setting-2 log-ratio is formed
  from logit differences and the stored LSE, never from log P.

Readings where the pages are silent (each is listed in the design notes):
* S_t = scale_t * Q_t K_t^T with scale_t = 1/sqrt(d_t) unless given.
* Causal masks are bottom-right aligned: key j is visible to query i iff
  j <= i + (N_K - N_Q).
* The loss reduction is left to the caller: the per-row upstream gradient g[i]
  multiplies row i, i.e. the backward returns the gradient of sum_i g[i] KL[i].
* Gradients (not printed on the pages) are the exact derivatives of that sum:
    setting 1: dS2 = g * (P2 - P1)
    setting 2: dS1 = g * P1 * ((S1 - LSE1) - (S2 - LSE2) - KL)
  and dQ_s = scale_s * dS_s K_s, dK_s = scale_s * dS_s^T Q_s; masked entries of
  dS are exactly zero.

All arithmetic is numpy float64.  Inputs (any float dtype, already rounded to
the precision the GPU receives) are converted exactly to float64 first.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "scores",
    "valid_mask",
    "head_forward",
    "head_backward",
    "head_backward_dk_rows",
    "head_dk_keys",
    "materialised_bytes",
    "pair_count",
]


def _f64(x) -> np.ndarray:
    """Exact widening to float64 (float32/float16 values are representable)."""
    return np.asarray(x, dtype=np.float64)


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else float(scale)


def valid_mask(rows: np.ndarray, n_q: int, n_k: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), n_k]: which keys each listed query row may attend to.

    Causal masking skips keys beyond the causal boundary (Method 1 of the
    technical summary); the boundary is read as bottom-right aligned.
    """
    cols = np.arange(n_k)[None, :]
    if not causal:
        return np.ones((len(rows), n_k), dtype=bool)
    return cols <= (np.asarray(rows)[:, None] + (n_k - n_q))


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * q k^T in float64 (the attention logits of one head)."""
    return scale * (_f64(q) @ _f64(k).T)


def _row_stats(S: np.ndarray, mask: np.ndarray):
    """Masked logits, LSE per row and log-probabilities (masked -> -inf)."""
    Sm = np.where(mask, S, -np.inf)
    m = Sm.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(Sm - m).sum(axis=1, keepdims=True)))[:, 0]
    logp = Sm - lse[:, None]
    return lse, logp


def _block_rows(rows: np.ndarray, block: int):
    for s in range(0, len(rows), block):
        yield rows[s:s + block]


def head_forward(q1, k1, q2, k2, causal: bool, scale1=None, scale2=None,
                 rows=None, block: int = 512):
    """KL[i], LSE1[i], LSE2[i] (natural log) for the listed query rows of one head.

    q_t: [N_Q, d_t], k_t: [N_K, d_t].  Returns float64 arrays of len(rows).
    KL is the definition sum_j P1 (log P1 - log P2) over visible keys.
    """
    q1, k1, q2, k2 = _f64(q1), _f64(k1), _f64(q2), _f64(k2)
    n_q, n_k = q1.shape[0], k1.shape[0]
    s1 = _default_scale(q1.shape[1], scale1)
    s2 = _default_scale(q2.shape[1], scale2)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    kl = np.empty(len(rows))
    lse1 = np.empty(len(rows))
    lse2 = np.empty(len(rows))
    pos = 0
    for rb in _block_rows(rows, block):
        mask = valid_mask(rb, n_q, n_k, causal)
        L1, logp1 = _row_stats(scores(q1[rb], k1, s1), mask)
        L2, logp2 = _row_stats(scores(q2[rb], k2, s2), mask)
        p1 = np.exp(logp1)  # exactly 0 where masked
        with np.errstate(invalid="ignore"):  # -inf - -inf on masked entries, discarded
            diff = np.where(mask, logp1 - logp2, 0.0)
        kl[pos:pos + len(rb)] = (p1 * diff).sum(axis=1)
        lse1[pos:pos + len(rb)] = L1
        lse2[pos:pos + len(rb)] = L2
        pos += len(rb)
    return kl, lse1, lse2


def _dS(setting: int, p1, p2, logp1, logp2, kl_rows, g_rows, mask):
    if setting == 1:
        dS = g_rows[:, None] * (p2 - p1)
    elif setting == 2:
        with np.errstate(invalid="ignore"):
            r = np.where(mask, logp1 - logp2, 0.0)
        dS = g_rows[:, None] * p1 * (r - kl_rows[:, None])
    else:
        raise ValueError("setting must be 1 or 2")
    return np.where(mask, dS, 0.0)


def head_backward(setting: int, q1, k1, q2, k2, causal: bool, g,
                  scale1=None, scale2=None, rows=None, block: int = 512, want_dk: bool = True):
    """Gradients of sum_i g[i] KL[i] for one head.

    setting 1 -> (dQ2[rows], dK2 contribution of those rows), P1 held fixed.
    setting 2 -> (dQ1[rows], dK1 contribution of those rows), P2 held fixed.
    With rows=None every row is used and dK is the full gradient.
    want_dk=False skips the dK product and returns None in its place (for
    key ranges whose [N_K, d] fp64 dK would not fit in memory).
    The KL used in setting 2 is recomputed here from the definition (the
    GPU path uses its stored forward value; both equal the same number).
    """
    q1, k1, q2, k2 = _f64(q1), _f64(k1), _f64(q2), _f64(k2)
    g = _f64(g)
    n_q, n_k = q1.shape[0], k1.shape[0]
    s1 = _default_scale(q1.shape[1], scale1)
    s2 = _default_scale(q2.shape[1], scale2)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    if setting not in (1, 2):
        raise ValueError("setting must be 1 or 2")
    qs, ks, ss = (q2, k2, s2) if setting == 1 else (q1, k1, s1)
    dq = np.empty((len(rows), qs.shape[1]))
    dk = np.zeros((n_k, ks.shape[1])) if want_dk else None
    pos = 0
    for rb in _block_rows(rows, block):
        mask = valid_mask(rb, n_q, n_k, causal)
        _, logp1 = _row_stats(scores(q1[rb], k1, s1), mask)
        _, logp2 = _row_stats(scores(q2[rb], k2, s2), mask)
        p1 = np.exp(logp1)
        p2 = np.exp(logp2)
        with np.errstate(invalid="ignore"):
            kl_rows = (p1 * np.where(mask, logp1 - logp2, 0.0)).sum(axis=1)
        dS = _dS(setting, p1, p2, logp1, logp2, kl_rows, g[rb], mask)
        dq[pos:pos + len(rb)] = ss * (dS @ ks)
        if want_dk:
            dk += ss * (dS.T @ qs[rb])
        pos += len(rb)
    return dq, dk


def head_backward_dk_rows(setting: int, q1, k1, q2, k2, causal: bool, g,
                          key_rows, scale1=None, scale2=None, block: int = 512):
    """Full gradient dK_s[key_rows] of sum_i g[i] KL[i] for one head.

    Only query rows that can see at least one of ``key_rows`` contribute, so
    for causal masks and tail key rows this touches only the last rows.
    """
    q1 = _f64(q1)
    n_q, n_k = q1.shape[0], _f64(k1).shape[0]
    key_rows = np.asarray(key_rows, dtype=np.int64)
    if causal:
        first = max(0, int(key_rows.min()) - (n_k - n_q))
        rows = np.arange(first, n_q)
    else:
        rows = np.arange(n_q)
    _, dk = head_backward(setting, q1, k1, q2, k2, causal, g, scale1, scale2,
                          rows=rows, block=block)
    return dk[key_rows]


def head_dk_keys(setting: int, q1, k1, q2, k2, causal: bool, g, key_rows, row_stats,
                 scale1=None, scale2=None, block: int = 512):
    """dK_s[key_rows] of sum_i g[i] KL[i] for one head, from the definition
    restricted to those key columns.

    ``row_stats`` = (kl, lse1, lse2) for EVERY query row of the head, as
    ``head_forward`` returns them (the LSE runs over all visible keys, so it
    cannot come from the selected columns).  Then for each selected key j:
    P_t[i, j] = exp(S_t[i, j] - LSE_t[i]) (technical summary, Method 2:
    probabilities regenerated from the stored LSE), dS as in ``_dS`` and
    dK_s[j] = scale_s * sum_i dS[i, j] Q_s[i].  Only len(key_rows) columns of
    the logits are formed, so the cost is O(N_Q * len(key_rows) * d) beyond
    the row statistics.
    """
    q1, k1, q2, k2 = _f64(q1), _f64(k1), _f64(q2), _f64(k2)
    g = _f64(g)
    n_q, n_k = q1.shape[0], k1.shape[0]
    s1 = _default_scale(q1.shape[1], scale1)
    s2 = _default_scale(q2.shape[1], scale2)
    if setting not in (1, 2):
        raise ValueError("setting must be 1 or 2")
    kl, lse1, lse2 = (_f64(x) for x in row_stats)
    if kl.shape != (n_q,) or lse1.shape != (n_q,) or lse2.shape != (n_q,):
        raise ValueError("row_stats must hold kl, lse1, lse2 for every query row")
    key_rows = np.asarray(key_rows, dtype=np.int64)
    qs, ss = (q2, s2) if setting == 1 else (q1, s1)
    dk = np.zeros((len(key_rows), qs.shape[1]))
    rows = np.arange(n_q)
    for rb in _block_rows(rows, block):
        mask = valid_mask(rb, n_q, n_k, causal)[:, key_rows]
        if not mask.any():
            continue
        with np.errstate(invalid="ignore"):
            logp1 = np.where(mask, scores(q1[rb], k1[key_rows], s1), -np.inf) - lse1[rb][:, None]
            logp2 = np.where(mask, scores(q2[rb], k2[key_rows], s2), -np.inf) - lse2[rb][:, None]
        p1 = np.exp(logp1)
        p2 = np.exp(logp2)
        dS = _dS(setting, p1, p2, logp1, logp2, kl[rb], g[rb], mask)
        dk += ss * (dS.T @ qs[rb])
    return dk


def pair_count(B: int, H: int, n_q: int, n_k: int, causal: bool) -> int:
    """Number of visible (query, key) pairs (the algorithmic work unit)."""
    if not causal:
        return B * H * n_q * n_k
    return B * H * (n_q * (n_q + 1) // 2 + n_q * (n_k - n_q))


def materialised_bytes(B: int, H: int, n_q: int, n_k: int,
                       bytes_per_elem: int = 2, n_dists: int = 2) -> int:
    """HBM bytes of the materialise-then-reduce baseline: both P1 and P2 stored.

    Technical summary, Problem statement, point 1 (quadratic memory footprint).
    """
    return n_dists * B * H * n_q * n_k * bytes_per_elem
