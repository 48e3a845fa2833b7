"""Error statistics used by the parity tests and the report -- test infrastructure only.

* max_rel_err: normwise max|x - ref| / max|ref| per tensor (an elementwise
  ratio is unbounded where ref is near zero).
* tail_sums: for each query row, the part of the unnormalised product that
  does NOT come from keys tied at the row maximum, tau[T, i] = sum over keys t
  farther than eps below the maximum of exp(S_Tt - rm_T) V[t, i], in float64.
  The pages explain the bias of plain BF16 through the rounding of the sum of
  the tied V values (P-bar = 1) in the presence of the remaining small terms,
  with predominantly negative V (section 3.4.4, "Why this creates systematic
  negative bias" and Claim 3).  Under round-to-nearest-even every step is odd
  in V, so for symmetric V the raw mean error is zero in expectation; the
  direction the rounding takes is set by the sign of that remainder.
* signed_error: the mean signed O error on tied rows, raw and oriented by the
  tail: s = -sign(tau) * (O_mode - O_exact).  When tau < 0 (the pages' case of
  negative V) s equals the raw error.  The sampling unit is the row (the mean
  over features of a row), so the standard error is across rows.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def max_rel_err(x, ref) -> float:
    x = np.asarray(x, F64)
    ref = np.asarray(ref, F64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(x - ref)))
    return float(np.max(np.abs(x - ref)) / den)


def tail_sums(q, k, v, causal=True, scale=None, eps=1e-3, q_pos=None):
    """tau [S, R, d] in float64 (see module docstring)."""
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    if q.ndim == 2:
        q, k, v = q[None], k[None], v[None]
    ns, r, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if q_pos is None:
        q_pos = np.arange(r)
    q_pos = np.broadcast_to(np.asarray(q_pos), (ns, r))
    s = np.matmul(q, k.transpose(0, 2, 1)) * scale
    if causal:
        keys = np.arange(k.shape[1])
        s = np.where(keys[None, None, :] > q_pos[:, :, None], -np.inf, s)
    rm = np.max(s, axis=-1, keepdims=True)
    w = np.exp(s - rm)
    w = np.where(rm - s <= eps, 0.0, w)
    return np.matmul(w, v)


def signed_error(o_mode, o_exact, tau, rows_mask):
    """Mean signed error on the rows in rows_mask.

    o_mode, o_exact, tau: [S, R, d]; rows_mask: [S, R] bool.
    Returns dict(rows, raw_mean, raw_se, tail_mean, tail_se).
    """
    o_mode = np.asarray(o_mode, F64)
    o_exact = np.asarray(o_exact, F64)
    err = (o_mode - o_exact)[rows_mask]          # [rows, d]
    t = np.asarray(tau, F64)[rows_mask]
    keep = t != 0
    oriented = np.where(keep, -np.sign(t) * err, 0.0)
    cnt = np.maximum(keep.sum(axis=-1), 1)
    row_tail = oriented.sum(axis=-1) / cnt
    row_raw = err.mean(axis=-1) if err.size else err.sum(axis=-1)
    nrow = err.shape[0]

    def mse(a):
        if len(a) == 0:
            return float("nan"), float("nan")
        if len(a) == 1:
            return float(a.mean()), float("nan")
        return float(a.mean()), float(a.std(ddof=1) / np.sqrt(len(a)))

    rm, rse = mse(row_raw)
    tm, tse = mse(row_tail)
    return dict(rows=int(nrow), raw_mean=rm, raw_se=rse, tail_mean=tm, tail_se=tse)
