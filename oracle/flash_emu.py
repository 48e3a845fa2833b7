"""Part B of the oracle: BF16-emulating tiled flash attention forward.

TEST INFRASTRUCTURE ONLY.  Follows, step by step and in the pages' order, the
tiled forward pass of flash attention with the online safe softmax (the
modified safe softmax of Algorithm 3 in section 3.4.5 of the paper-graph-ui
summary of arXiv 2510.04212), rounding every intermediate the way a BF16
kernel with FP32 accumulation does.  Rows are independent, so any subset of
query rows can be emulated (all rows for small shapes, tied rows plus a sample
for long sequences).

Per query row T and per key tile j of width bn (keys t, masked when t > T in
causal attention), starting from M = M2 = m = -inf, l = 0, Obar = 0:

 1. x_t = fp32(q_T . k_t)  (the dot of BF16 vectors in float64, then rounded);
    S_t = fp32(x_t * fp32(scale)).  S is the softmax input the pages call S.
 2. Merge the tile's scores into the running top two of the row, as a
    multiset: M is the largest score so far, M2 the second largest (equal to M
    when the maximum occurs twice).  The tie flag is fp32(M - M2) <= fp32(eps)
    -- "rs = rowsum(rm - S <= eps) > 1" of section 3.4.5, kept exactly across
    tiles, so the final flag equals the untiled rule.
 3. Shift m: plain modes use m = M.  The tie-aware mode uses
    m = fp32(beta * M) when the flag is set and M > 0, m = 0 when the flag is
    set and M < 0, and m = M otherwise (section 3.4.5, the two "where" lines).
 4. alpha = exp(m_old - m_new) in FP32 (0 on the first tile).
 5. p_t = exp(fp32(S_t - m_new)) in FP32.
 6. P-bar_t = bf16(p_t) in the BF16 modes.  In the FP32-output mode the
    product uses the high-precision P-bar: hi + lo with hi = bf16(p),
    lo = bf16(p - hi)  (section 3.4.4 reports that an FP32 P-bar V product
    alone is enough to stabilise training).
 7. l = fp32(alpha * l + sum_t P-bar_t) and Obar = fp32(alpha * Obar +
    sum_t P-bar_t v_t): FP32 accumulation, each tile's sum formed exactly and
    rounded once.  l sums the same P-bar that multiplies V, as in the pages'
    O = Obar / rowsum(P-bar).
 8. Epilogue.  BF16 modes: Obar is rounded to BF16 once (section 3.4.4 defines
    the low-precision product as an FP32 dot product whose final result is
    rounded to BF16) and O = bf16(fp32(bf16(Obar) / l)).  FP32-output mode: O = fp32(Obar / l).
    LSE = fp32(m + log l).  The output flag is the flag after the last tile.

Readings where the pages leave a step open (listed with reasons in the design
notes): the single BF16 rounding of Obar after FP32 accumulation over all tiles
(step 8), l from the same rounded P-bar (step 7), the hi/lo P-bar of the FP32
output mode (step 6), and the row-global running tie flag (step 2).

With exact=True every rounding is switched off and all arithmetic is float64;
the result must then equal plain attention in every mode (the shift invariance
of section 3.4.5).  That is one of the pins in tests/test_oracle_flash_emu.py.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import bf16_rne, f32

F64 = np.float64
F32 = np.float32

MODES = ("bf16_out", "fp32_out", "tie_aware_softmax")


class _Round:
    """The rounding steps of the BF16 kernel, or identities in exact mode."""

    def __init__(self, exact: bool):
        self.exact = exact

    def r32(self, x):
        return np.asarray(x, F64) if self.exact else f32(x).astype(F64)

    def bf(self, x):
        return np.asarray(x, F64) if self.exact else bf16_rne(f32(x)).astype(F64)

    def exp(self, x):
        x = np.asarray(x, F64)
        if self.exact:
            return np.exp(x)
        with np.errstate(under="ignore", over="ignore"):
            return np.exp(x.astype(F32)).astype(F64)

    def log(self, x):
        x = np.asarray(x, F64)
        if self.exact:
            with np.errstate(divide="ignore"):
                return np.log(x)
        with np.errstate(divide="ignore"):
            return np.log(x.astype(F32)).astype(F64)


@dataclass
class EmuResult:
    o: np.ndarray          # [S, R, d]  output (BF16 values or FP32 values, as float64)
    lse: np.ndarray        # [S, R]
    flag: np.ndarray       # [S, R] bool, final tie flag
    row_max: np.ndarray    # [S, R] M, the row maximum of S
    row_max2: np.ndarray   # [S, R] M2, second largest (multiset)
    m_final: np.ndarray    # [S, R] the shift in force after the last tile
    obar: np.ndarray       # [S, R, d] FP32 accumulator before the epilogue
    l: np.ndarray          # [S, R] FP32 row sum of P-bar
    n_pbar_one: np.ndarray  # [S, R] number of entries whose P-bar rounds to 1 in BF16
    max_pbar_flagged: np.ndarray  # [S, R] max P-bar over the tiles processed while the flag was set (-1 if none)
    obar_one: np.ndarray   # [S, R, d] the part of obar from those entries (P-bar taken as 1)


def pbar_one_threshold() -> float:
    """The smallest FP32 value t for which P-bar = bf16(fp32(exp(t))) is 1.

    P-bar is formed in FP32 and rounded to BF16 (nearest, ties to even).  BF16
    below 1 has spacing 2^-8, so the FP32 value rounds to 1 exactly when it is
    at least 1 - 2^-9 (the halfway point goes to the even 1.0); with a
    correctly rounded FP32 exp that is exp(t) >= 1 - 2^-9 - 2^-25, just above
    ln(1 - 2^-9) = -0.0019550...  The FP32 values t near it are 2^-32 apart;
    float64 exp rounded to FP32 decides each of them.
    """
    target = np.float32(1.0 - 2.0 ** -9)
    rn = lambda t: np.float32(np.exp(np.float64(t)))
    t = np.float32(np.log(np.float64(target)))
    while rn(t) < target:
        t = np.nextafter(t, np.float32(0))
    while rn(np.nextafter(t, np.float32(-1))) >= target:
        t = np.nextafter(t, np.float32(-1))
    return float(t)


def _top2_multiset(s):
    """Largest and second largest along the last axis (multiset), -inf padded."""
    if s.shape[-1] == 1:
        return s[..., 0], np.full(s.shape[:-1], -np.inf)
    part = -np.partition(-s, 1, axis=-1)[..., :2]
    return part[..., 0], part[..., 1]


def flash_forward(q, k, v, mode="bf16_out", causal=True, scale=None, bn=64,
                  beta=2.0, eps=1e-3, q_pos=None, exact=False) -> EmuResult:
    """Emulated tiled forward.

    q: [S, R, d] query rows (BF16 values), k, v: [S, N, d] (BF16 values).
    q_pos: [R] or [S, R] query positions of the rows (default arange(R), i.e.
    all rows of an N = R sequence); used for the causal mask.
    Leading dims other than one slice dim must be flattened by the caller.
    """
    if mode not in MODES:
        raise ValueError(f"unknown mode {mode!r}")
    rd = _Round(exact)
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    if q.ndim == 2:
        q, k, v = q[None], k[None], v[None]
    ns, r, d = q.shape
    n = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if q_pos is None:
        q_pos = np.arange(r)
    q_pos = np.broadcast_to(np.asarray(q_pos), (ns, r))
    s_scale = rd.r32(scale)
    eps_r = rd.r32(eps)
    beta_r = rd.r32(beta)
    tie_mode = mode == "tie_aware_softmax"
    hp = mode == "fp32_out"

    big_m = np.full((ns, r), -np.inf)
    big_m2 = np.full((ns, r), -np.inf)
    m = np.full((ns, r), -np.inf)
    el = np.zeros((ns, r))
    obar = np.zeros((ns, r, v.shape[2]))
    n_one = np.zeros((ns, r), np.int64)
    obar_one = np.zeros_like(obar)
    one_thr = pbar_one_threshold()
    flag = np.zeros((ns, r), bool)
    max_after = np.full((ns, r), -1.0)

    for j0 in range(0, n, bn):
        j1 = min(n, j0 + bn)
        if causal and j0 > q_pos.max():
            break
        kt = k[:, j0:j1]
        vt = v[:, j0:j1]
        x = rd.r32(np.matmul(q, kt.transpose(0, 2, 1)))
        s = rd.r32(x * s_scale)
        if causal:
            keys = np.arange(j0, j1)
            s = np.where(keys[None, None, :] > q_pos[:, :, None], -np.inf, s)
        # step 2: running top two (multiset) and the tie flag
        t1, t2 = _top2_multiset(s)
        cand = np.stack([big_m, big_m2, t1, t2], axis=-1)
        big_m, big_m2 = _top2_multiset(cand)
        with np.errstate(invalid="ignore"):
            gap = rd.r32(big_m - big_m2)
        flag = np.isfinite(big_m2) & (gap <= eps_r)
        # step 3: the shift
        if tie_mode:
            m_new = np.where(flag & (big_m > 0), rd.r32(beta_r * big_m),
                             np.where(flag & (big_m < 0), 0.0, big_m))
        else:
            m_new = big_m.copy()
        # step 4: rescale factor for the earlier tiles
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(m), rd.exp(rd.r32(m - m_new)), 0.0)
        # rows whose keys in this tile are all masked keep their state
        active = np.isfinite(t1)
        alpha = np.where(active, alpha, 1.0)
        m_use = np.where(active, m_new, 0.0)
        # step 5-6: probabilities and the P-bar that enters the product
        with np.errstate(invalid="ignore"):
            d_arg = rd.r32(s - m_use[..., None])
            p = rd.exp(d_arg)
        p = np.where(np.isfinite(s), p, 0.0)
        # the entries whose P-bar rounds to 1 in BF16 (the P-bar = 1 additions
        # of section 3.4.4): decided on d = S - m against the threshold of a
        # correctly rounded FP32 exp, the same entries in every mode
        with np.errstate(invalid="ignore"):
            ones = (np.isfinite(s) & (d_arg >= one_thr)).astype(F64)
        if hp and not rd.exact:
            hi = rd.bf(p)
            lo = rd.bf(rd.r32(p - hi))
            pbar = hi + lo
        elif hp:
            pbar = p
        else:
            pbar = rd.bf(p)
        n_one += np.sum(ones, axis=-1).astype(np.int64)
        tile_max = np.max(pbar, axis=-1)
        max_after = np.where(flag & active, np.maximum(max_after, tile_max), max_after)
        # step 7: FP32 accumulation, one rounding per tile
        el = np.where(active, rd.r32(alpha * el + np.sum(pbar, axis=-1)), el)
        obar_new = rd.r32(alpha[..., None] * obar + np.matmul(pbar, vt))
        obar = np.where(active[..., None], obar_new, obar)
        one_new = rd.r32(alpha[..., None] * obar_one + np.matmul(ones, vt))
        obar_one = np.where(active[..., None], one_new, obar_one)
        m = np.where(active, m_new, m)

    # step 8: epilogue
    with np.errstate(divide="ignore", invalid="ignore"):
        if hp or rd.exact:
            o = rd.r32(obar / el[..., None])
        else:
            ob = rd.bf(obar)
            o = rd.bf(rd.r32(ob / el[..., None]))
        lse = rd.r32(m + rd.log(el))
    return EmuResult(o=o, lse=lse, flag=flag, row_max=big_m, row_max2=big_m2,
                     m_final=m, obar=obar, l=el, n_pbar_one=n_one,
                     max_pbar_flagged=max_after, obar_one=obar_one)


def tie_flags_untiled(q, k, causal=True, scale=None, eps=1e-3, q_pos=None, return_gap=False):
    """The pages' untiled rule: rs = rowsum(rm - S <= eps), flag = rs > 1.

    S is rounded exactly as in flash_forward step 1.  Returns (flag, rs), and
    with return_gap also the gap between the largest and second largest score
    (multiset; inf where a row has a single unmasked key).
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    if q.ndim == 2:
        q, k = q[None], k[None]
    ns, r, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if q_pos is None:
        q_pos = np.arange(r)
    q_pos = np.broadcast_to(np.asarray(q_pos), (ns, r))
    s = f32(f32(np.matmul(q, k.transpose(0, 2, 1))).astype(F64) * f32(scale).astype(F64)).astype(F64)
    if causal:
        keys = np.arange(k.shape[1])
        s = np.where(keys[None, None, :] > q_pos[:, :, None], -np.inf, s)
    rm = np.max(s, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore"):
        diff = f32(rm - s).astype(F64)
    rs = np.sum(np.isfinite(s) & (diff <= float(f32(eps))), axis=-1)
    if not return_gap:
        return rs > 1, rs
    top1, top2 = _top2_multiset(s)
    with np.errstate(invalid="ignore"):
        gap = np.where(np.isfinite(top2), f32(top1 - top2).astype(F64), np.inf)
    return rs > 1, rs, gap, top1


def tie_top2_untiled(q, k, causal=True, scale=None, eps=1e-3, q_pos=None, chunk=512):
    """The untiled rule of tie_flags_untiled for one (batch, head) slice, stated
    through the row's two largest scores: rs > 1 exactly when the second
    largest score (multiset) lies within eps of the largest, because
    fp32(rm - S) grows as S falls.  S is rounded as in flash_forward step 1.

    q: [R, d] query rows, k: [N, d] keys (BF16 values); q_pos as in
    tie_flags_untiled.  Rows are processed `chunk` at a time, so long
    sequences need only chunk x N scores at once.  Returns (flag [R] bool,
    gap [R] = fp32(M - M2), inf for a row with one visible key, M [R]).
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    r, d = q.shape
    n = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    q_pos = np.arange(r) if q_pos is None else np.asarray(q_pos)
    s32 = F32(scale)
    eps32 = F32(eps)
    keys = np.arange(n)
    flag = np.zeros(r, bool)
    gap = np.empty(r, F32)
    top = np.empty(r, F32)
    kt = np.ascontiguousarray(k.T)
    for r0 in range(0, r, chunk):
        r1 = min(r, r0 + chunk)
        s = (q[r0:r1] @ kt).astype(F32) * s32        # fp32(fp32(q.k) * fp32(scale))
        if causal:
            s[keys[None, :] > q_pos[r0:r1, None]] = -np.inf
        m1 = s.max(axis=1)
        at_max = s == m1[:, None]
        n_max = at_max.sum(axis=1)
        s[at_max] = -np.inf
        m2 = np.where(n_max >= 2, m1, s.max(axis=1))
        with np.errstate(invalid="ignore"):
            g = np.where(np.isfinite(m2), m1 - m2, F32(np.inf)).astype(F32)
        gap[r0:r1] = g
        top[r0:r1] = m1
        flag[r0:r1] = np.isfinite(m2) & (g <= eps32)
    return flag, gap, top
