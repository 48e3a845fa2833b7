"""Pins of oracle/stats.py: hand-computed values that a plausible slip in any
of its functions (a wrong denominator, a per-element instead of per-row unit,
ddof = 0, a sign, row instead of cluster resampling) would change.

The tail sums are checked on the hand-built tie of tests/golden/
hand_tie_example.json (every query 64 e0, K0 = K1 = e0, K2 = 0.25 e0,
scale 1/8): row 2 scores (8, 8, 2), keys 0 and 1 tied at the maximum, so its
tail is exp(2 - 8) V[2] (paper-graph-ui summary of arXiv 2510.04212, section
3.4.4, the remainder beside the P-bar = 1 entries in "Why this creates
systematic negative bias").
"""
import math

import numpy as np
import pytest

from oracle import stats as st


# ---- max_rel_err: max |x - ref| / max |ref| ---------------------------------

def test_max_rel_err_two_elements():
    # |x - ref| = (0.5, 6); max |ref| = 4 -> 1.5.  The mean of |ref| (2.75) or
    # an elementwise ratio (max(1/3, 1.5)) would not give 1.5 here, nor would a
    # denominator of max |x| (2).
    assert st.max_rel_err([1.0, 2.0], [1.5, -4.0]) == 1.5
    assert st.max_rel_err([1.0, -4.5], [1.5, -4.0]) == 0.5 / 4.0


def test_max_rel_err_zero_reference_is_absolute():
    assert st.max_rel_err([0.25, -0.5], [0.0, 0.0]) == 0.5


def test_max_rel_err_is_normwise_not_elementwise():
    # a tiny reference element with a relatively large error does not dominate
    assert st.max_rel_err([1.0, 1e-6 + 1e-7], [1.0, 1e-6]) == pytest.approx(1e-7, rel=1e-9)


# ---- tail_sums on the hand-built tie -----------------------------------------

def _hand_tie(d=64):
    q = np.zeros((3, d))
    q[:, 0] = 64.0
    k = np.zeros((3, d))
    k[0, 0] = k[1, 0] = 1.0
    k[2, 0] = 0.25
    v = np.zeros((3, d))
    v[:, 0] = (-2.296875, -2.40625, -2.0)
    v[:, 1] = -v[:, 0]
    return q, k, v


def test_tail_sums_hand_tie_closed_form():
    q, k, v = _hand_tie()
    tau = st.tail_sums(q, k, v, causal=True, scale=0.125)[0]
    e6 = math.exp(-6.0)
    # row 0 sees only key 0 (its own maximum); row 1 sees the two tied keys
    assert np.all(tau[0] == 0.0) and np.all(tau[1] == 0.0)
    assert tau[2, 0] == pytest.approx(-2.0 * e6, rel=1e-15)
    assert tau[2, 1] == pytest.approx(2.0 * e6, rel=1e-15)
    assert np.all(tau[2, 2:] == 0.0)
    # without the mask every row sees all three keys
    tnc = st.tail_sums(q, k, v, causal=False, scale=0.125)[0]
    for r in range(3):
        assert tnc[r, 0] == pytest.approx(-2.0 * e6, rel=1e-15)


def test_tail_sums_eps_excludes_keys_within_eps_of_the_maximum():
    # key 2 raised to S = 8 - 2^-11 (within eps = 1e-3 of the maximum): tied,
    # so row 2 has no tail; at 8 - 2^-9 (beyond eps) it is the tail again
    q, k, v = _hand_tie()
    k[2, 0] = 1.0 - 2.0 ** -11 / 8.0
    assert np.all(st.tail_sums(q, k, v, scale=0.125)[0][2] == 0.0)
    k[2, 0] = 1.0 - 2.0 ** -9 / 8.0
    tau = st.tail_sums(q, k, v, scale=0.125)[0]
    assert tau[2, 0] == pytest.approx(-2.0 * math.exp(-2.0 ** -9), rel=1e-15)


# ---- signed_error: row unit, tail orientation, ddof = 1 ----------------------

def _three_rows():
    # four rows of d = 2; row 3 is not in the mask
    o_exact = np.zeros((1, 4, 2))
    err = np.array([[0.1, -0.3], [0.2, 0.2], [-0.5, 0.1], [9.0, 9.0]])
    tau = np.array([[1.0, -1.0], [-2.0, 0.0], [3.0, 3.0], [1.0, 1.0]])
    mask = np.array([[True, True, True, False]])
    return o_exact + err[None], o_exact, tau[None], mask


def test_signed_error_hand_rows():
    o, ref, tau, mask = _three_rows()
    r = st.signed_error(o, ref, tau, mask)
    assert r["rows"] == 3
    # oriented -sign(tau)*err: row 0 (-0.1, -0.3) -> -0.2; row 1 (0.2, tau 0
    # left out) -> 0.2; row 2 (0.5, -0.1) -> 0.2.  Mean 1/15; deviations
    # (-4, 2, 2)/15, sum of squares 24/225, / (n - 1) = 12/225, SE = 2/15.
    assert r["tail_mean"] == pytest.approx(1.0 / 15.0, rel=1e-12)
    assert r["tail_se"] == pytest.approx(2.0 / 15.0, rel=1e-12)
    # raw row means (-0.1, 0.2, -0.2): mean -1/30; deviations (-2, 7, -5)/30,
    # sum of squares 78/900, / 2 = 39/900, SE = sqrt(39/900/3) = sqrt(13)/30
    assert r["raw_mean"] == pytest.approx(-1.0 / 30.0, rel=1e-12)
    assert r["raw_se"] == pytest.approx(math.sqrt(13.0) / 30.0, rel=1e-12)


def test_signed_error_row_without_tail_is_left_out_of_the_tail_statistic():
    o, ref, tau, mask = _three_rows()
    tau[0, 1] = 0.0   # row 1 now has tau = 0 in both features
    r = st.signed_error(o, ref, tau, mask)
    # tail rows: -0.2 and 0.2 -> mean 0, SE = sqrt(0.08 / 2) = 0.2
    assert r["tail_mean"] == pytest.approx(0.0, abs=1e-15)
    assert r["tail_se"] == pytest.approx(0.2, rel=1e-12)
    assert r["rows"] == 3 and r["raw_mean"] == pytest.approx(-1.0 / 30.0, rel=1e-12)


def test_signed_error_negative_tail_is_the_raw_error():
    # with tau < 0 everywhere (the pages' negative-V case) tail = raw
    rng = np.random.default_rng(3)
    o = rng.standard_normal((1, 50, 8))
    ref = rng.standard_normal((1, 50, 8))
    tau = -np.abs(rng.standard_normal((1, 50, 8))) - 0.1
    mask = np.ones((1, 50), bool)
    r = st.signed_error(o, ref, tau, mask)
    assert r["tail_mean"] == pytest.approx(r["raw_mean"], rel=1e-12)
    assert r["tail_se"] == pytest.approx(r["raw_se"], rel=1e-12)


# ---- ratio_ci: cluster bootstrap of |mean plain| / |mean tie| ----------------

def test_ratio_ci_without_spread_is_the_point_ratio():
    plain = np.full(40, -2e-5)
    tie = np.full(40, 1e-6)
    r = st.ratio_ci(plain, tie, groups=np.arange(40) // 4, n_boot=200)
    assert r["ratio"] == pytest.approx(20.0, rel=1e-12)
    assert r["lo"] == pytest.approx(20.0, rel=1e-12) and r["hi"] == pytest.approx(20.0, rel=1e-12)
    assert r["clusters"] == 10


def test_ratio_ci_uses_absolute_means():
    r = st.ratio_ci(np.full(10, 3.0), np.full(10, -0.5), groups=np.arange(10), n_boot=50)
    assert r["ratio"] == pytest.approx(6.0, rel=1e-12)


def test_ratio_ci_matches_the_delta_method_for_large_samples():
    # independent rows, plain ~ N(-10, 1), tie ~ N(1, 1), 40000 clusters of one
    # row: the ratio's standard deviation is about
    # 10 * sqrt((0.005/10)^2 + (0.005/1)^2) = 0.0502, so the 95% interval is
    # about 10 +- 0.098
    rng = np.random.default_rng(11)
    n = 40000
    plain = -10.0 + rng.standard_normal(n)
    tie = 1.0 + rng.standard_normal(n)
    r = st.ratio_ci(plain, tie, groups=np.arange(n), n_boot=1000, seed=5)
    half = 1.96 * r["ratio"] * math.sqrt((1.0 / math.sqrt(n) / 10.0) ** 2 + (1.0 / math.sqrt(n)) ** 2)
    assert r["lo"] == pytest.approx(r["ratio"] - half, abs=0.25 * half)
    assert r["hi"] == pytest.approx(r["ratio"] + half, abs=0.25 * half)


def test_ratio_ci_resamples_clusters_not_rows():
    # 500 clusters of 8 identical rows carry the information of 500 rows: the
    # interval equals that of one row per cluster (same seed), and is wider
    # than a row-level bootstrap of the 4000 rows would give
    rng = np.random.default_rng(2)
    p1 = -10.0 + rng.standard_normal(500)
    t1 = 1.0 + rng.standard_normal(500)
    one = st.ratio_ci(p1, t1, groups=np.arange(500), n_boot=400, seed=9)
    eight = st.ratio_ci(np.repeat(p1, 8), np.repeat(t1, 8), groups=np.repeat(np.arange(500), 8),
                        n_boot=400, seed=9)
    assert eight["lo"] == pytest.approx(one["lo"], rel=1e-12)
    assert eight["hi"] == pytest.approx(one["hi"], rel=1e-12)
    rows = st.ratio_ci(np.repeat(p1, 8), np.repeat(t1, 8), groups=np.arange(4000), n_boot=400, seed=9)
    assert (rows["hi"] - rows["lo"]) < 0.6 * (eight["hi"] - eight["lo"])


def test_ratio_ci_rejects_mismatched_inputs():
    with pytest.raises(ValueError):
        st.ratio_ci(np.zeros(3), np.zeros(4), np.zeros(3))
