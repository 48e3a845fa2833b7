"""Inputs whose tie test sits one FP32 ulp on either side of eps (test helper).

With d = 64 and scale 1/8 (exact), a query row T holds 2^-2 in feature 0 and
ones in features 1..n; key a holds 2^-3 in feature 0 and key b holds 2^-3 in
feature 0 and -2^(i - 30) in feature j for the set bits i of an integer g, so
that S_a = 2^-8 and S_b = 2^-8 - g 2^-33 exactly.  Every term and every
partial sum of the dot products is a multiple of 2^-29 below 2^-5 in
magnitude, hence exact in FP32 in any summation order.  eps = fp32(1e-3) =
8589935 2^-33, so g = 8589934 (eps - 1 ulp) must set the flag and g = 8589936
(eps + 1 ulp) must not (the rule flag = fp32(M - M2) <= fp32(eps)).  All other
keys and query rows are zero (their scores all tie at 0).
"""
import numpy as np

EPS_INT = 8589935                      # fp32(1e-3) = EPS_INT * 2^-33
GAPS = (EPS_INT - 1, EPS_INT + 1)      # flagged, not flagged
T, KEY_A, KEY_B, N, D = 7, 2, 5, 8, 64


def boundary_inputs():
    """q, k, v [1, 2, N, D] float32 (BF16-exact): head 0 with gap eps - 1 ulp,
    head 1 with gap eps + 1 ulp at query row T; expected flags of row T."""
    assert np.float32(1e-3).view(np.uint32) & 0x7FFFFF | 0x800000 == EPS_INT
    q = np.zeros((1, 2, N, D), np.float32)
    k = np.zeros((1, 2, N, D), np.float32)
    rng = np.random.default_rng(5)
    v = np.round(rng.standard_normal((1, 2, N, D)) * 8).astype(np.float32) / 8
    for h, g in enumerate(GAPS):
        bits = [i for i in range(40) if (g >> i) & 1]
        assert len(bits) < D and min(bits) >= 1
        q[0, h, T, 0] = 2.0 ** -2
        q[0, h, T, 1:1 + len(bits)] = 1.0
        k[0, h, KEY_A, 0] = 2.0 ** -3
        k[0, h, KEY_B, 0] = 2.0 ** -3
        for j, i in enumerate(bits):
            k[0, h, KEY_B, 1 + j] = -(2.0 ** (i - 30))
    return q, k, v, (True, False)
