"""Pins of oracle/attention64.py (Part A, float64 attention)."""
import math

import numpy as np
import pytest

from oracle import attention64 as a64


def _loops_forward(q, k, v, causal, scale):
    """Scalar loops: weights exp(s) / sum exp(s) without any max subtraction."""
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i in range(n):
        w = []
        for j in range(k.shape[0]):
            if causal and j > i:
                w.append(0.0)
                continue
            s = sum(float(q[i, c]) * float(k[j, c]) for c in range(d)) * scale
            w.append(math.exp(s))
        z = sum(w)
        lse[i] = math.log(z)
        for j, wj in enumerate(w):
            o[i] += (wj / z) * v[j]
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d", [(1, 3), (5, 4), (8, 2)])
def test_forward_matches_scalar_loops(causal, n, d):
    rng = np.random.default_rng(n * 10 + d)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, lse = a64.attention_fwd(q[None], k[None], v[None], causal=causal, scale=0.7)
    o2, lse2 = _loops_forward(q, k, v, causal, 0.7)
    np.testing.assert_allclose(o[0], o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0], lse2, rtol=0, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(0)
    n, d = 9, 4
    v = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    zq = np.zeros((n, d))
    o, lse = a64.attention_fwd(zq, k, v, causal=True, scale=1.0)
    # zero queries: every visible key has the same weight -> running means
    want = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, want, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), atol=1e-14)
    o, _ = a64.attention_fwd(zq, k, v, causal=False, scale=1.0)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), atol=1e-14)
    # causal row 0 sees one key: O[0] = V[0], and its query gets no gradient
    q = rng.standard_normal((n, d))
    o, _ = a64.attention_fwd(q, k, v, causal=True, scale=0.5)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    g = a64.attention_bwd(q, k, v, rng.standard_normal((n, d)), causal=True, scale=0.5)
    assert np.abs(g["dq"][0]).max() < 1e-15


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((64, 16)) * 3 for _ in range(3))
    _, _, p = a64.fwd_slice(q, k, v, True, 0.25)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    assert np.all(np.triu(p, 1) == 0)


@pytest.mark.parametrize("causal", [True, False])
def test_gradients_match_finite_differences(causal):
    rng = np.random.default_rng(2)
    n, d = 6, 3
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    scale = 0.8

    def loss(q_, k_, v_):
        o, _ = a64.attention_fwd(q_, k_, v_, causal=causal, scale=scale)
        return float(np.sum(do * o))

    g = a64.attention_bwd(q, k, v, do, causal=causal, scale=scale)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = {"dq": 0, "dk": 1, "dv": 2}[name]
            args_p[pos] = xp
            args_m[pos] = xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g[name], num, atol=2e-8, rtol=1e-6)


def test_delta_identity():
    """rowsum(dO o O) equals rowsum(dP o P) (section 3.4.2)."""
    rng = np.random.default_rng(4)
    q, k, v, do = (rng.standard_normal((32, 8)) for _ in range(4))
    g = a64.attention_bwd(q, k, v, do, causal=True, scale=0.35)
    np.testing.assert_allclose(g["delta"], g["delta_p"], atol=1e-12)


def test_delta_conditioning_bounds():
    """cond_p and cond_o bound |delta_p| and |delta| (triangle inequality), and
    reduce to the single product on a row with one visible key (causal row 0):
    cond_p = |dO_0 . v_0|, cond_o = sum_i |dO_0i v_0i|."""
    rng = np.random.default_rng(6)
    n, d = 24, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    g = a64.bwd_slice(q, k, v, do, True, 0.3)
    assert np.all(np.abs(g["delta_p"]) <= g["cond_p"] * (1 + 1e-12))
    assert np.all(np.abs(g["delta"]) <= g["cond_o"] * (1 + 1e-12))
    assert np.isclose(g["cond_p"][0], abs(do[0] @ v[0]), rtol=1e-13)
    assert np.isclose(g["cond_o"][0], np.sum(np.abs(do[0] * v[0])), rtol=1e-13)
    # equal weights (zero queries): cond_o of the last row is the mean of |dO| . |v_t|
    z = a64.bwd_slice(np.zeros((n, d)), k, v, do, True, 0.3)
    want = np.mean(np.abs(v) @ np.abs(do[-1]))
    assert np.isclose(z["cond_o"][-1], want, rtol=1e-13)


def test_dq_error_identity():
    """dQ_hp - dQ_lp = scale * diag(delta_lp - delta_hp) (P K)  (section 3.4.3)."""
    rng = np.random.default_rng(5)
    n, d = 16, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    scale = 0.3
    o_hp, _ = a64.attention_fwd(q, k, v, causal=True, scale=scale)
    o_lp = o_hp + 1e-2 * rng.standard_normal(o_hp.shape)   # a perturbed (low-precision) O
    g_hp = a64.attention_bwd(q, k, v, do, causal=True, scale=scale, o=o_hp)
    g_lp = a64.attention_bwd(q, k, v, do, causal=True, scale=scale, o=o_lp)
    _, _, p = a64.fwd_slice(q, k, v, True, scale)
    want = scale * (g_lp["delta"] - g_hp["delta"])[:, None] * (p @ k)
    np.testing.assert_allclose(g_hp["dq"] - g_lp["dq"], want, atol=1e-13)
    # dK and dV: dV does not use delta; dK changes by scale * (diag(delta_lp - delta_hp) P)^T Q
    np.testing.assert_allclose(g_hp["dv"], g_lp["dv"], atol=1e-14)
    want_k = scale * (p * (g_lp["delta"] - g_hp["delta"])[:, None]).T @ q
    np.testing.assert_allclose(g_hp["dk"] - g_lp["dk"], want_k, atol=1e-13)


def test_flop_count():
    assert a64.flops_fwd_bwd(1, 16, 8192, 128) == 962072674304


@pytest.mark.parametrize("causal", [True, False])
def test_row_chunked_reference_equals_whole_slice(causal):
    rng = np.random.default_rng(9)
    n, d = 70, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    r = a64.slice_reference(q, k, v, do, causal=causal, scale=0.4, chunk=16)
    o, lse, _ = a64.fwd_slice(q, k, v, causal, 0.4)
    g = a64.bwd_slice(q, k, v, do, causal, 0.4)
    np.testing.assert_allclose(r["o"], o, atol=1e-13)
    np.testing.assert_allclose(r["lse"], lse, atol=1e-13)
    for key in ("dq", "dk", "dv", "delta", "delta_p", "cond_p", "cond_o"):
        np.testing.assert_allclose(r[key], g[key], atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_sampled_rows_equal_whole_slice(causal):
    """The row-sampled reference (query rows for O, LSE, delta, dQ; key rows
    for dK, dV, summed over every query that sees the key) equals the same
    rows of the whole-slice reference; rows in arbitrary order, chunks that
    split both loops."""
    rng = np.random.default_rng(12)
    n, d = 75, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    qr = np.array([74, 0, 3, 40, 41, 1, 63])
    kr = np.array([70, 5, 0, 74, 33])
    r = a64.sampled_reference(q, k, v, do, qr, kr, causal=causal, scale=0.4, chunk=4)
    o, lse, _ = a64.fwd_slice(q, k, v, causal, 0.4)
    g = a64.bwd_slice(q, k, v, do, causal, 0.4)
    np.testing.assert_allclose(r["o"], o[qr], atol=1e-13)
    np.testing.assert_allclose(r["lse"], lse[qr], atol=1e-13)
    np.testing.assert_allclose(r["delta"], g["delta"][qr], atol=1e-12)
    np.testing.assert_allclose(r["dq"], g["dq"][qr], atol=1e-12)
    np.testing.assert_allclose(r["dk"], g["dk"][kr], atol=1e-12)
    np.testing.assert_allclose(r["dv"], g["dv"][kr], atol=1e-12)
