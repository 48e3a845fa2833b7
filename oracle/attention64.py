"""Part A of the oracle: plain attention in float64 -- test infrastructure only.

This is the "exact result" every mode is compared with.  All three modes compute
the same function in exact arithmetic, because softmax is unchanged by a
per-row shift (paper-graph-ui summary of arXiv 2510.04212, section 3.4.5,
"Mathematical equivalence in exact arithmetic").

Forward (section 3.4.4, the three-line definition of P-bar, O-bar and O):
    S = scale * Q K^T, causal entries (key index > query index) set to -inf
    P = softmax of each row of S
    O = P V,  LSE = log sum_t exp(S_t)
Backward (section 3.4.2 "Failure is linked to the computation of delta" and
section 3.4.3 "Derivation of the gradient error"):
    dV = P^T dO,  dP = dO V^T,  delta = rowsum(dO o O)
    dS = P o (dP - delta),  dQ = scale * dS K,  dK = scale * dS^T Q
The pages give dQ only; dK and dV are the standard gradients of the same
product (the plainest reading).

Inputs are numpy arrays shaped [..., N, d] holding the values the kernel sees
(BF16 values stored as float32, or FP32 dO).  Every (batch, head) slice is
handled on its own so memory stays at a few N x N float64 matrices.

Pinned by tests/test_oracle_attention64.py: brute-force scalar loops on tiny
shapes, closed forms (zero queries give running means, row 0 of a causal
product copies V[0]), softmax rows summing to one, central finite differences
of sum(dO o O) for every gradient, the delta identity and the dQ identity;
the row-chunked and row-sampled references against the whole-slice one.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _slices(x):
    lead = x.shape[:-2]
    return lead, int(np.prod(lead)) if lead else 1


def _scores(q, k, causal, scale):
    s = (q @ k.T) * F64(scale)
    if causal:
        n = s.shape[0]
        s[np.triu_indices(n, 1, s.shape[1])] = -np.inf
    return s


def _softmax_rows(s):
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def fwd_slice(q, k, v, causal, scale):
    """One (batch, head) slice: returns O [N,d], LSE [N], P [N,N] (float64)."""
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    s = _scores(q, k, causal, scale)
    p, lse = _softmax_rows(s)
    return p @ v, lse, p


def bwd_slice(q, k, v, do, causal, scale, o=None):
    """One slice of the backward.  Returns dict with dq, dk, dv, delta, delta_p,
    cond_p, cond_o.

    delta uses O (the given one, or the exact O when o is None); delta_p is the
    equivalent rowsum(dP o P), which the pages report as the stabilising
    alternative (section 3.2 and section 3.4.2).  cond_p = rowsum(P o |dP|) and
    cond_o = sum_i |dO_i| (P |V|)_i are the magnitudes the two sums are built
    from: a computation of delta_p (or of rowsum(dO o P V)) with relative
    rounding u per operation errs by a small multiple of u times them.
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    do = np.asarray(do, F64)
    o_exact, _, p = fwd_slice(q, k, v, causal, scale)
    o_used = o_exact if o is None else np.asarray(o, F64)
    dv = p.T @ do
    dp = do @ v.T
    delta = np.sum(do * o_used, axis=-1)
    delta_p = np.sum(dp * p, axis=-1)
    cond_p = np.sum(np.abs(dp) * p, axis=-1)
    cond_o = np.sum(np.abs(do) * (p @ np.abs(v)), axis=-1)
    ds = p * (dp - delta[:, None])
    dq = F64(scale) * (ds @ k)
    dk = F64(scale) * (ds.T @ q)
    return dict(dq=dq, dk=dk, dv=dv, delta=delta, delta_p=delta_p, cond_p=cond_p, cond_o=cond_o,
                p=p, o=o_exact)


def attention_fwd(q, k, v, causal=True, scale=None):
    """Batched forward over leading dims.  Returns (O, LSE) in float64."""
    q = np.asarray(q)
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    lead, nsl = _slices(q)
    n = q.shape[-2]
    qs, ks, vs = (x.reshape(nsl, x.shape[-2], x.shape[-1]) for x in (q, k, v))
    o = np.empty((nsl, n, vs.shape[-1]), F64)
    lse = np.empty((nsl, n), F64)
    for i in range(nsl):
        o[i], lse[i], _ = fwd_slice(qs[i], ks[i], vs[i], causal, scale)
    return o.reshape(*lead, n, vs.shape[-1]), lse.reshape(*lead, n)


def attention_bwd(q, k, v, do, causal=True, scale=None, o=None):
    """Batched backward.  Returns dict of float64 arrays dq, dk, dv, delta, delta_p,
    cond_p, cond_o (see bwd_slice).

    o: optional output to form delta = rowsum(dO o O) with (e.g. the BF16 O of
    a kernel); by default the exact O is used.
    """
    q = np.asarray(q)
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    lead, nsl = _slices(q)
    n = q.shape[-2]
    rs = lambda x: None if x is None else np.asarray(x).reshape(nsl, x.shape[-2], x.shape[-1])
    qs, ks, vs, dos, os_ = rs(q), rs(k), rs(v), rs(do), rs(o)
    out = {key: [] for key in ("dq", "dk", "dv", "delta", "delta_p", "cond_p", "cond_o")}
    for i in range(nsl):
        r = bwd_slice(qs[i], ks[i], vs[i], dos[i], causal, scale,
                      None if os_ is None else os_[i])
        for key in out:
            out[key].append(r[key])
    res = {}
    for key, vals in out.items():
        arr = np.stack(vals)
        res[key] = arr.reshape(*lead, *arr.shape[1:])
    return res


def flops_fwd_bwd(b, h, n, d, causal=True):
    """Algorithmic FLOPs of forward + backward: 2 products forward, 5 backward
    (the S recompute, dP, dV, dK, dQ), each 2*N*N*d, halved when causal."""
    f = 7 * 2 * b * h * n * n * d
    return f // 2 if causal else f


def slice_reference(q, k, v, do=None, causal=True, scale=None, o_for_delta=None, chunk=1024):
    """Forward and backward of one (batch, head) slice in float64, query rows
    taken `chunk` at a time so long sequences fit in memory.

    Query rows are independent in the forward, in delta and in dQ; dK and dV
    are sums over query rows and are accumulated chunk by chunk.  Same
    definitions as fwd_slice / bwd_slice (pinned against them in the tests).
    o_for_delta: the O used in delta = rowsum(dO o O) (default: the exact O).
    Returns dict(o, lse, dq, dk, dv, delta, delta_p, cond_p, cond_o) of float64
    arrays (the last three as in bwd_slice).
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    n, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = dict(o=np.empty((n, v.shape[1])), lse=np.empty(n))
    if do is not None:
        do = np.asarray(do, F64)
        out.update(dq=np.empty((n, d)), dk=np.zeros_like(k), dv=np.zeros_like(v), delta=np.empty(n),
                   delta_p=np.empty(n), cond_p=np.empty(n), cond_o=np.empty(n))
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        kend = r1 if causal else k.shape[0]
        s = (q[r0:r1] @ k[:kend].T) * F64(scale)
        if causal:
            rows = np.arange(r0, r1)[:, None]
            s = np.where(np.arange(kend)[None, :] > rows, -np.inf, s)
        p, lse = _softmax_rows(s)
        o = p @ v[:kend]
        out["o"][r0:r1] = o
        out["lse"][r0:r1] = lse
        if do is None:
            continue
        g = do[r0:r1]
        o_used = o if o_for_delta is None else np.asarray(o_for_delta[r0:r1], F64)
        dp = g @ v[:kend].T
        delta = np.sum(g * o_used, axis=-1)
        ds = p * (dp - delta[:, None])
        out["dq"][r0:r1] = F64(scale) * (ds @ k[:kend])
        out["dk"][:kend] += F64(scale) * (ds.T @ q[r0:r1])
        out["dv"][:kend] += p.T @ g
        out["delta"][r0:r1] = delta
        out["delta_p"][r0:r1] = np.sum(dp * p, axis=-1)
        out["cond_p"][r0:r1] = np.sum(np.abs(dp) * p, axis=-1)
        out["cond_o"][r0:r1] = np.sum(np.abs(g) * (p @ np.abs(v[:kend])), axis=-1)
    return out


def sampled_reference(q, k, v, do, q_rows, k_rows, causal=True, scale=None, chunk=256):
    """Forward and backward outputs of selected rows of one (batch, head)
    slice in float64, for sequences too long for whole-slice references.

    Query rows (O, LSE, delta, dQ) need only their own row of S.  A key row
    j of dK = scale * dS^T Q and dV = P^T dO sums over every query i that sees
    key j (i >= j when causal); each such query's row of P (and its delta) is
    formed whole, `chunk` queries at a time, and only the columns of the
    selected keys enter the sums.  Same definitions as fwd_slice / bwd_slice
    (pinned against slice_reference in the tests).
    Returns dict(o, lse, delta, dq) for q_rows and dict(dk, dv) for k_rows,
    float64, in the order given.
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    do = np.asarray(do, F64)
    n, d = q.shape
    scale = F64(1.0 / np.sqrt(d) if scale is None else scale)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    keys = np.arange(k.shape[0])

    def rows_state(rows):
        s = (q[rows] @ k.T) * scale
        if causal:
            s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
        p, lse = _softmax_rows(s)
        o = p @ v
        delta = np.sum(do[rows] * o, axis=-1)
        return p, lse, o, delta

    out = dict(o=np.empty((len(q_rows), v.shape[1])), lse=np.empty(len(q_rows)),
               delta=np.empty(len(q_rows)), dq=np.empty((len(q_rows), d)),
               dk=np.zeros((len(k_rows), d)), dv=np.zeros((len(k_rows), v.shape[1])))
    for c0 in range(0, len(q_rows), chunk):
        sel = slice(c0, min(len(q_rows), c0 + chunk))
        rows = q_rows[sel]
        p, lse, o, delta = rows_state(rows)
        dp = do[rows] @ v.T
        ds = p * (dp - delta[:, None])
        out["o"][sel], out["lse"][sel], out["delta"][sel] = o, lse, delta
        out["dq"][sel] = scale * (ds @ k)
    if len(k_rows):
        first = int(k_rows.min()) if causal else 0
        for r0 in range(first, n, chunk):
            rows = np.arange(r0, min(n, r0 + chunk))
            p, _, _, delta = rows_state(rows)
            pk = p[:, k_rows]
            dpk = do[rows] @ v[k_rows].T
            dsk = pk * (dpk - delta[:, None])
            out["dk"] += scale * (dsk.T @ q[rows])
            out["dv"] += pk.T @ do[rows]
    return out
