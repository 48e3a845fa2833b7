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
  over features of a row), so the standard error is across rows.  Features
  with tau = 0 carry no orientation and are left out of a row's tail mean; a
  row with tau = 0 in every feature is left out of the tail statistic.
* ratio_ci: the plain / tie-aware ratio of the mean tail-oriented error with a
  percentile bootstrap confidence interval.  Rows of one repetition share
  their keys and values, so whole repetitions (clusters of rows) are
  resampled, and a resample takes the same repetitions in both modes.
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


def row_values(o_mode, o_exact, tau, rows_mask):
    """Per-row statistics on the rows in rows_mask (the sampling units):
    (tail, raw, kept).  tail[r] = mean over the features with tau != 0 of
    -sign(tau) * (O_mode - O_exact); raw[r] = mean over all features of
    O_mode - O_exact; kept[r] = the row has at least one feature with tau != 0
    (rows without one carry no tail-oriented value)."""
    o_mode = np.asarray(o_mode, F64)
    o_exact = np.asarray(o_exact, F64)
    err = (o_mode - o_exact)[rows_mask]          # [rows, d]
    t = np.asarray(tau, F64)[rows_mask]
    keep = t != 0
    oriented = np.where(keep, -np.sign(t) * err, 0.0)
    cnt = keep.sum(axis=-1)
    tail = oriented.sum(axis=-1) / np.maximum(cnt, 1)
    raw = err.mean(axis=-1) if err.size else err.sum(axis=-1)
    return tail, raw, cnt > 0


def _mean_se(a):
    if len(a) == 0:
        return float("nan"), float("nan")
    if len(a) == 1:
        return float(a.mean()), float("nan")
    return float(a.mean()), float(a.std(ddof=1) / np.sqrt(len(a)))


def signed_error(o_mode, o_exact, tau, rows_mask):
    """Mean signed error on the rows in rows_mask.

    o_mode, o_exact, tau: [S, R, d]; rows_mask: [S, R] bool.
    Returns dict(rows, raw_mean, raw_se, tail_mean, tail_se): means over rows
    and standard errors across rows (sample standard deviation, n - 1).  Rows
    whose tail is zero in every feature enter the raw statistic only.
    """
    tail, raw, kept = row_values(o_mode, o_exact, tau, rows_mask)
    rm, rse = _mean_se(raw)
    tm, tse = _mean_se(tail[kept])
    return dict(rows=int(len(raw)), raw_mean=rm, raw_se=rse, tail_mean=tm, tail_se=tse)


def ratio_ci(plain, tie, groups, n_boot=2000, level=0.95, seed=0):
    """|mean(plain)| / |mean(tie)| with a percentile bootstrap interval.

    plain, tie: per-row values of the two modes on the same rows (paired);
    groups: the cluster (repetition) of each row.  A resample draws as many
    clusters as there are, with replacement, and takes all rows of each drawn
    cluster in both modes; its ratio is |sum plain| / |sum tie| over those rows
    (the row counts cancel).  Returns dict(ratio, lo, hi, n_boot, clusters).
    """
    plain = np.asarray(plain, F64)
    tie = np.asarray(tie, F64)
    groups = np.asarray(groups)
    if not (plain.shape == tie.shape == groups.shape) or plain.ndim != 1:
        raise ValueError("plain, tie and groups must be 1-d arrays of one length")
    _, g = np.unique(groups, return_inverse=True)
    ng = int(g.max()) + 1 if g.size else 0
    sp = np.bincount(g, weights=plain, minlength=ng)
    st = np.bincount(g, weights=tie, minlength=ng)
    with np.errstate(divide="ignore"):
        ratio = float(abs(sp.sum()) / abs(st.sum()))
    rng = np.random.Generator(np.random.PCG64(seed))
    boots = np.empty(n_boot)
    chunk = max(1, min(n_boot, (1 << 24) // max(ng, 1)))
    for b0 in range(0, n_boot, chunk):
        b1 = min(n_boot, b0 + chunk)
        idx = rng.integers(0, ng, size=(b1 - b0, ng))
        with np.errstate(divide="ignore"):
            boots[b0:b1] = np.abs(sp[idx].sum(axis=1)) / np.abs(st[idx].sum(axis=1))
    a = (1.0 - level) / 2.0
    lo, hi = np.quantile(boots, [a, 1.0 - a])
    return dict(ratio=ratio, lo=float(lo), hi=float(hi), n_boot=int(n_boot), clusters=ng)
