"""Pins of oracle/flash_emu.py (Part B, the BF16-emulating tiled forward)."""
import json
import os

import numpy as np
import pytest

from oracle import attention64 as a64
from oracle import flash_emu as fe
from oracle import stats as st
from oracle.numerics import bf16_rne, f32, is_bf16
from synth.inputs import generate, generate_reps, to_bf16_values, workload

GOLD = os.path.join(os.path.dirname(__file__), "golden")
MODES = fe.MODES


def _rand_bf16(rng, *shape, s=1.0):
    return to_bf16_values((rng.standard_normal(shape) * s).astype(np.float32))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,bn", [(37, 8), (64, 64), (100, 32), (50, 50)])
def test_exact_skeleton_equals_plain_attention(mode, causal, n, bn):
    """With rounding switched off, every mode is plain attention (softmax is
    unchanged by a per-row shift, section 3.4.5); bn = n is the untiled run."""
    rng = np.random.default_rng(n + bn)
    d = 16
    q = _rand_bf16(rng, n, d, s=6.0)
    k = _rand_bf16(rng, n, d)
    v = _rand_bf16(rng, n, d)
    # force a few exact ties (duplicated keys) so the tie rule fires
    k[5] = k[2]
    k[9] = k[2]
    q[9] = 8 * q[9]
    scale = 0.25
    r = fe.flash_forward(q, k, v, mode=mode, causal=causal, scale=scale, bn=bn, exact=True)
    o, lse = a64.attention_fwd(q, k, v, causal=causal, scale=scale)
    np.testing.assert_allclose(r.o[0], o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(r.lse[0], lse, atol=1e-12, rtol=0)


@pytest.mark.parametrize("bn", [16, 64, 128])
def test_online_flags_equal_untiled_rule(bn):
    x = generate(workload(1))
    q, k = x.q[0], x.k[0]
    fl_u, rs = fe.tie_flags_untiled(q, k)
    for mode in MODES:
        r = fe.flash_forward(q, k, x.v[0], mode=mode, bn=bn)
        assert np.array_equal(r.flag, fl_u)
    # every forced row has at least two tied maxima
    assert fl_u.sum() >= 1
    x3 = generate(workload(3, b=1, h=2, n=256))
    for h in range(2):
        fl3, _ = fe.tie_flags_untiled(x3.q[0, h], x3.k[0, h])
        r = fe.flash_forward(x3.q[0, h], x3.k[0, h], x3.v[0, h], bn=bn)
        assert np.array_equal(r.flag[0], fl3[0])


def test_tie_flag_eps_boundary():
    """Gaps of 2^-10 (< 1e-3) tie, gaps of 2^-9 (> 1e-3) do not."""
    d = 64
    q = np.zeros((4, d), np.float32)
    q[:, 0] = 8.0
    q[:, 1] = 8.0
    k = np.zeros((4, d), np.float32)
    k[0, 0] = 1.0                      # S = 1
    k[1, 0] = 1.0
    k[1, 1] = -2.0 ** -10              # S = 1 - 2^-10
    k[2, 0] = 1.0
    k[2, 1] = -2.0 ** -9               # S = 1 - 2^-9
    k[3, 0] = 1.0
    k[3, 1] = -2.0 ** -9
    assert np.all(is_bf16(k)) and np.all(is_bf16(q))
    r = fe.flash_forward(q, k, np.ones((4, d), np.float32), causal=True, scale=1 / 8)
    assert r.flag[0].tolist() == [False, True, True, True]
    k2 = k.copy()
    k2[1] = k[2]                       # key 0 is the unique maximum, the rest 2^-9 below
    r = fe.flash_forward(q, k2, np.ones((4, d), np.float32), causal=True, scale=1 / 8)
    assert r.flag[0].tolist() == [False, False, False, False]
    k2[0] = k[2]                       # now all four keys are equal
    r = fe.flash_forward(q, k2, np.ones((4, d), np.float32), causal=True, scale=1 / 8)
    assert r.flag[0].tolist() == [False, True, True, True]


def test_hand_built_tie_example():
    g = json.load(open(os.path.join(GOLD, "hand_tie_example.json")))
    d = 64
    q = np.zeros((3, d), np.float32)
    q[:, 0] = 64.0
    k = np.zeros((3, d), np.float32)
    k[0, 0] = k[1, 0] = 1.0
    k[2, 0] = 0.25
    v = np.zeros((3, d), np.float32)
    v[:, 0] = [-2.296875, -2.40625, -2.0]
    v[:, 1] = -v[:, 0]
    for mode in ("bf16_out", "tie_aware_softmax"):
        r = fe.flash_forward(q, k, v, mode=mode, scale=1 / 8)
        for row in range(3):
            assert r.o[0, row, 0] == g["expected"][mode][f"row{row}"], (mode, row)
            assert r.o[0, row, 1] == -g["expected"][mode][f"row{row}"]
        assert r.flag[0].astype(int).tolist() == [g["flags"][f"row{i}"] for i in range(3)]
    o, _ = a64.attention_fwd(q, k, v, causal=True, scale=1 / 8)
    for row in range(3):
        assert abs(o[row, 0] - g["expected"]["exact"][f"row{row}"]) < 1e-15
    r = fe.flash_forward(q, k, v, mode="fp32_out", scale=1 / 8)
    np.testing.assert_allclose(r.o[0, :, 0], o[:, 0], rtol=1e-5)


def test_plain_mode_pbar_is_one_at_every_maximum():
    """Plain safe softmax: P-bar = 1 exactly at each maximum (section 3.4.4)."""
    x = generate(workload(1))
    q, k, v = x.q[0], x.k[0], x.v[0]
    r = fe.flash_forward(q, k, v, mode="bf16_out")
    fl, rs = fe.tie_flags_untiled(q, k, eps=0.0)   # exact-equality count of maxima
    assert np.all(r.n_pbar_one >= rs)
    assert np.all(r.n_pbar_one[fl] >= 2)


def test_tie_mode_guarantee_no_pbar_of_one_once_flagged():
    """Tie-aware mode: max P-bar < 1 in every tile processed while the flag is
    set (section 3.4.5), except rows whose maximum is 0 or whose shifted
    maximum still rounds to 1 (|rm| * (beta-1) below ~2e-3)."""
    x = generate_reps(workload(1), 8)
    b = x.q.shape[0]
    q, k, v = (a.reshape(b, 128, 64) for a in (x.q, x.k, x.v))
    r = fe.flash_forward(q, k, v, mode="tie_aware_softmax", bn=32)
    flagged = r.max_pbar_flagged >= 0
    ok = np.abs(r.row_max) > 4e-3
    assert flagged.sum() > 100
    assert np.all(r.max_pbar_flagged[flagged & ok] < 1.0)


def test_never_fired_rows_are_bitwise_plain():
    x = generate_reps(workload(1), 4)
    b = x.q.shape[0]
    q, k, v = (a.reshape(b, 128, 64) for a in (x.q, x.k, x.v))
    rp = fe.flash_forward(q, k, v, mode="bf16_out", bn=32)
    rt = fe.flash_forward(q, k, v, mode="tie_aware_softmax", bn=32)
    never = rt.max_pbar_flagged < 0
    assert never.sum() > 50 and (~never).sum() > 50
    assert np.array_equal(rp.o[never], rt.o[never])
    assert np.array_equal(rp.lse[never], rt.lse[never])
    assert not np.array_equal(rp.o[~never], rt.o[~never])


@pytest.mark.parametrize("mode", MODES)
def test_odd_symmetry_in_v(mode):
    """Round-to-nearest-even is odd, so O(-V) = -O(V) bit for bit."""
    x = generate(workload(1))
    q, k, v = x.q[0], x.k[0], x.v[0]
    a = fe.flash_forward(q, k, v, mode=mode)
    b = fe.flash_forward(q, k, -v, mode=mode)
    assert np.array_equal(a.o, -b.o)


@pytest.mark.parametrize("mode,tol", [("bf16_out", 2e-2), ("tie_aware_softmax", 2e-2), ("fp32_out", 1e-4)])
def test_emulator_within_the_stated_tolerances(mode, tol):
    x = generate(workload(2, b=1, h=2, n=256))
    for h in range(2):
        q, k, v = x.q[0, h], x.k[0, h], x.v[0, h]
        r = fe.flash_forward(q, k, v, mode=mode)
        o, lse = a64.attention_fwd(q, k, v)
        assert st.max_rel_err(r.o[0], o) <= tol
        if mode != "fp32_out":
            assert np.all(is_bf16(r.o))
    if mode == "fp32_out":
        assert st.max_rel_err(r.o[0], o) <= 1e-5


def test_underflow_of_large_tied_maximum_gives_nan():
    """(beta - 1) * rm beyond the FP32 exp range: l underflows, the row is NaN
    (the unconditional shift's failure the pages warn about, section 3.4.5)."""
    d = 64
    q = np.zeros((2, d), np.float32)
    q[:, 0] = 128.0
    k = np.zeros((2, d), np.float32)
    k[:, 0] = 8.0                                # S = 128 for both keys, tied
    v = np.ones((2, d), np.float32)
    r = fe.flash_forward(q, k, v, mode="tie_aware_softmax", scale=1 / 8)
    assert r.flag[0, 1] and np.all(np.isnan(r.o[0, 1]))
    r = fe.flash_forward(q, k, v, mode="tie_aware_softmax", scale=1 / 8, beta=1.5)
    assert np.all(np.isfinite(r.o[0, 1]))


def _signed(wl, reps, modes):
    x = generate_reps(wl, reps)
    b = x.q.shape[0]
    q, k, v = (a.reshape(b, wl.n, wl.d) for a in (x.q, x.k, x.v))
    o64 = np.stack([a64.fwd_slice(q[i], k[i], v[i], True, wl.scale)[0] for i in range(b)])
    tau = st.tail_sums(q, k, v, scale=wl.scale)
    out = {}
    for mode in modes:
        r = fe.flash_forward(q, k, v, mode=mode, scale=wl.scale)
        out[mode] = st.signed_error(r.o, o64, tau, r.flag)
    return out


def test_sign_claim_plain_biased_tie_aware_not():
    """Tied rows (P-bar = 1 at several keys): plain BF16 rounds the product
    towards the tail (negative oriented mean); the tie-aware softmax removes it."""
    res = _signed(workload(1), 400, ("bf16_out", "tie_aware_softmax", "fp32_out"))
    p, t, f = res["bf16_out"], res["tie_aware_softmax"], res["fp32_out"]
    assert p["tail_mean"] < -5 * p["tail_se"]
    assert abs(t["tail_mean"]) < 3 * t["tail_se"]
    assert abs(f["tail_mean"]) < 1e-3 * abs(p["tail_mean"])


def test_sign_claim_negative_values_paper_condition():
    """With mostly negative V (V - 2) the raw plain-BF16 error on tied rows is
    negative (Claim 3) and the tie-aware mode shrinks it."""
    res = _signed(workload(1, v_shift=-2.0), 300, ("bf16_out", "tie_aware_softmax"))
    p, t = res["bf16_out"], res["tie_aware_softmax"]
    assert p["raw_mean"] < -5 * p["raw_se"]
    assert abs(t["raw_mean"]) < 0.5 * abs(p["raw_mean"])


def test_flag_one_ulp_either_side_of_eps():
    """Exact inputs whose top-two score gap is fp32(eps) -/+ one ulp (2^-33):
    the untiled rule and the tiled emulator (one tile, and 2-key tiles whose
    running top two meet across tiles) flag the first and not the second."""
    from eps_boundary import T, boundary_inputs
    q, k, v, expect = boundary_inputs()
    for h in range(2):
        fl, _, gap, _ = fe.tie_flags_untiled(q[0, h], k[0, h], scale=0.125, return_gap=True)
        assert gap[0][T] == np.float64(np.float32(1e-3)) + (-1 if h == 0 else 1) * 2.0 ** -33
        assert bool(fl[0][T]) == expect[h]
        for bn in (64, 2):
            r = fe.flash_forward(q[0, h][None], k[0, h][None], v[0, h][None], mode="tie_aware_softmax",
                                 causal=True, scale=0.125, bn=bn)
            assert bool(r.flag[0][T]) == expect[h]
            assert np.array_equal(r.flag[0], fl[0])


@pytest.mark.parametrize("causal", [True, False])
def test_top2_statement_equals_the_rs_rule(causal):
    """tie_top2_untiled (the rule through the two largest scores) against the
    pages' count form rs = rowsum(rm - S <= eps) > 1: forced ties (config 1),
    natural ties of sharp rows (config 3's Q x4), the one-ulp eps boundary
    inputs and eps = 0."""
    from eps_boundary import boundary_inputs
    cases = []
    x = generate(workload(1))
    cases.append((x.q[0, 0], x.k[0, 0], 0.125, 1e-3))
    x3 = generate(workload(3, b=1, h=2, n=300))
    cases += [(x3.q[0, h], x3.k[0, h], 0.125, 1e-3) for h in range(2)]
    cases.append((x3.q[0, 0], x3.k[0, 0], 0.125, 0.0))
    qb, kb, _, _ = boundary_inputs()
    cases += [(qb[0, h], kb[0, h], 0.125, 1e-3) for h in range(qb.shape[1])]
    for q, k, scale, eps in cases:
        fl, rs, gap, top = fe.tie_flags_untiled(q, k, causal=causal, scale=scale, eps=eps, return_gap=True)
        f2, g2, t2 = fe.tie_top2_untiled(q, k, causal=causal, scale=scale, eps=eps, chunk=37)
        assert np.array_equal(f2, fl[0])
        assert np.array_equal(t2.astype(np.float64), top[0])
        fin = np.isfinite(gap[0])
        assert np.array_equal(np.isfinite(g2), fin)
        assert np.array_equal(g2[fin].astype(np.float64), gap[0][fin])
    assert sum(int(fe.tie_top2_untiled(q, k, causal=causal, scale=s, eps=e)[0].sum())
               for q, k, s, e in cases) > 10


def test_pbar_one_threshold_is_the_bf16_rounding_boundary():
    """At the threshold t, exp rounded to FP32 is 1 - 2^-9, which BF16 rounds
    (ties to even) to 1; one FP32 step lower it is 1 - 2^-9 - 2^-24, which
    rounds to 1 - 2^-8.  t is the first FP32 value (spacing 2^-32 there) at or
    above ln(1 - 2^-9 - 2^-25) = -0.00195506...
    (numpy's own FP32 exp is not correctly rounded there: it gives 1 - 2^-9
    one step below t, which is why the count uses this threshold.)"""
    from oracle.numerics import bf16_rne
    t = np.float32(fe.pbar_one_threshold())
    below = np.nextafter(t, np.float32(-1))
    for x, fp32, b16 in ((t, 1 - 2.0 ** -9, 1.0), (below, 1 - 2.0 ** -9 - 2.0 ** -24, 1 - 2.0 ** -8)):
        e = np.float32(np.exp(np.float64(x)))
        assert e == np.float32(fp32)
        assert bf16_rne(e) == np.float32(b16)
    assert 0 <= float(t) - np.log1p(-2.0 ** -9 - 2.0 ** -25) < 2.0 ** -32


@pytest.mark.parametrize("bn", [32, 64])
def test_pbar_one_count_matches_the_rounded_pbar(bn):
    """The count equals the number of entries of the rounded P-bar that are
    exactly 1 in the plain mode (no entry of these inputs sits within the FP32
    exp error of the threshold), and the FP32-output mode counts the same
    entries (same running maximum)."""
    x = generate_reps(workload(1), 4)
    b = x.q.shape[0]
    q, k, v = (a.reshape(b, 128, 64) for a in (x.q, x.k, x.v))
    r = fe.flash_forward(q, k, v, mode="bf16_out", bn=bn)
    rh = fe.flash_forward(q, k, v, mode="fp32_out", bn=bn)
    assert np.array_equal(r.n_pbar_one, rh.n_pbar_one)
    # recount: the rounded P-bar of each tile, with the row maximum known
    # after the tile as the shift
    cnt = np.zeros((b, 128), np.int64)
    big = np.full((b, 128), -np.inf)
    for j0 in range(0, 128, bn):
        x_ = f32(np.matmul(q.astype(np.float64), k[:, j0:j0 + bn].transpose(0, 2, 1).astype(np.float64)))
        s_ = f32(x_.astype(np.float64) * np.float64(np.float32(0.125))).astype(np.float64)
        s_ = np.where(np.arange(j0, j0 + bn)[None, None, :] > np.arange(128)[None, :, None], -np.inf, s_)
        big = np.maximum(big, s_.max(axis=-1))
        with np.errstate(invalid="ignore"):
            pb = bf16_rne(np.exp(f32(s_ - big[..., None])))
        cnt += np.sum(pb == 1.0, axis=-1)
    assert np.array_equal(cnt, r.n_pbar_one)
    fl, rs = fe.tie_flags_untiled(q, k, eps=0.0)
    assert np.all(r.n_pbar_one >= rs) and np.all(r.n_pbar_one[fl] >= 2)
    assert r.n_pbar_one.sum() > b * 128


def test_pbar_one_part_of_obar_on_the_hand_tie():
    """The hand-built tie (tests/golden/hand_tie_example.json): in the plain
    mode the P-bar = 1 entries of rows 1 and 2 are keys 0 and 1, whose V sum
    -2.296875 - 2.40625 = -4.703125 is exact in FP32, and row 0's is key 0; in
    the tie-aware mode the shift 2 * 8 leaves no entry at 1 on the tied rows."""
    d = 64
    q = np.zeros((3, d), np.float32)
    q[:, 0] = 64.0
    k = np.zeros((3, d), np.float32)
    k[0, 0] = k[1, 0] = 1.0
    k[2, 0] = 0.25
    v = np.zeros((3, d), np.float32)
    v[:, 0] = (-2.296875, -2.40625, -2.0)
    v[:, 1] = -v[:, 0]
    r = fe.flash_forward(q, k, v, mode="bf16_out", scale=1 / 8)
    assert list(r.n_pbar_one[0]) == [1, 2, 2]
    assert list(r.obar_one[0, :, 0]) == [-2.296875, -4.703125, -4.703125]
    assert list(r.obar_one[0, :, 1]) == [2.296875, 4.703125, 4.703125]
    assert np.all(r.obar_one[0, :, 2:] == 0.0)
    t = fe.flash_forward(q, k, v, mode="tie_aware_softmax", scale=1 / 8)
    assert list(t.n_pbar_one[0]) == [1, 0, 0]
    assert list(t.obar_one[0, :, 0]) == [-2.296875, 0.0, 0.0]
    h = fe.flash_forward(q, k, v, mode="fp32_out", scale=1 / 8)
    assert np.array_equal(h.n_pbar_one, r.n_pbar_one) and np.array_equal(h.obar_one, r.obar_one)
