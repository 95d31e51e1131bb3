"""Numeric identities the HIP kernels rely on to reproduce the contract's fp32 roundings by a
cheaper route, checked on the CPU with IEEE numpy arithmetic (no GPU, no oracle).

Adam's bias-corrected moments are m1 / bc1 and v1 / bc2, each rounded once to fp32. The
kernels compute them as RN32(RN64(x * y)) with y = RN64(1 / bc) formed on the host: the fp64
product is within 2^-52 (relative) of the quotient, and the quotient of two fp32 values is
never closer than about 2^-48 (relative) to a midpoint between floats unless it is a float,
so the final rounding always lands where RN32(x / bc) does.
"""
import numpy as np


def _via_recip64(a, b):
    with np.errstate(all="ignore"):
        return (a.astype(np.float64) * (1.0 / b.astype(np.float64))).astype(np.float32)


def _same(x, y):
    return (x == y) | (np.isnan(x) & np.isnan(y))


def test_division_by_fp64_reciprocal_is_correctly_rounded_random():
    rng = np.random.default_rng(11)
    n = 2_000_000
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-150, 120, n))).astype(np.float32)
    b = np.abs(rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    b = np.maximum(b, np.float32(1e-30))
    a[:6] = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45]
    with np.errstate(all="ignore"):
        ref = a / b
    assert _same(_via_recip64(a, b), ref).all()


def test_division_by_adam_bias_corrections_every_significand():
    """Every fp32 significand in [1, 2) divided by the bias corrections of two betas at a few
    steps (first steps, where bc is far from 1, and later ones)."""
    sig = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(0x3F800000)).view(np.float32)
    for beta, steps in ((0.9, (1, 2, 7, 50)), (0.999, (1, 3, 100, 1000))):
        for t in steps:
            bc = np.float32(1.0 - beta ** t)
            y = 1.0 / np.float64(bc)
            a = sig * np.float32(2.0 ** -9)
            got = (a.astype(np.float64) * y).astype(np.float32)
            assert np.array_equal(got, a / bc), (beta, t)


def test_division_by_recip64_subnormal_and_overflowing_quotients():
    b = np.float32(0.1)
    a = np.array([1e-45, 3e-45, 1.17e-38, 1.2e-38, 3.4e38, -3.4e38, 3.0e37], np.float32)
    with np.errstate(all="ignore"):
        assert _same(_via_recip64(a, np.full_like(a, b)), a / b).all()


def _fma32(a, b, c):
    """RN32(a * b + c) for fp32 inputs: the product of two fp32 values and its sum with an
    fp32 value of at most 2^4 times its size is exact in fp64 here (|a| <= 15), so one
    rounding to fp32 is the fused multiply-add."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def test_int4_dequant_by_one_fma_is_the_rounded_product():
    """The INT4 dequantization computes fl(q * s) as RN(u * s - 8 s) with u = q + 8: for every
    code q in [-8, 7] and scales across the fp32 range below 2^125 (subnormal, tiny, typical,
    large), including scales with full 24-bit significands where q * s itself rounds."""
    rng = np.random.default_rng(5)
    n = 200_000
    s = (rng.random(n) + 1.0) * np.exp2(rng.integers(-149, 125, n))
    s = s.astype(np.float32)
    s[:6] = [1e-45, 3e-39, 1.17549435e-38, 0.1, 1.0, np.float32(2.0 ** 124 * 1.9999999)]
    s = s[np.abs(s) < np.float32(2.0 ** 125)]
    for q in range(-8, 8):
        u = np.full(s.shape, q + 8, np.float32)
        c = (np.float32(-8.0) * s).astype(np.float32)
        assert np.isfinite(c).all()
        got = _fma32(u, s, c)
        want = (np.float32(q) * s).astype(np.float32)
        assert np.array_equal(got.view(np.uint32) & 0x7FFFFFFF, want.view(np.uint32) & 0x7FFFFFFF) \
            and np.array_equal(got, want), q


# ---------------------------------------------------------------------------------------
# The rounding's alpha fold. With alpha = 2^k (-126 < k <= 0) and U not written, the
# back-projection takes U * (1/s) as S * fl(alpha * (1/s)) instead of fl(alpha * S) * (1/s).
# Scaling by a power of two is exact outside the subnormal range, so the two agree bit for bit
# whenever alpha * S is normal or zero and alpha * (1/s) is normal, zero or infinite; where
# alpha * S is subnormal they differ by less than 2^-21 (one rounding of at most 2^-150, times
# a reciprocal below 2^128, plus the final roundings of the two products).

def _unfolded(S, inv, alpha):
    with np.errstate(all="ignore"):
        return ((alpha * S).astype(np.float32) * inv).astype(np.float32)


def _folded(S, inv, alpha):
    with np.errstate(all="ignore"):
        return (S * (alpha * inv).astype(np.float32)).astype(np.float32)


def test_alpha_fold_is_exact_outside_the_subnormal_range():
    rng = np.random.default_rng(23)
    n = 2_000_000
    S = (rng.standard_normal(n) * np.exp2(rng.integers(-100, 20, n))).astype(np.float32)
    inv = np.abs(rng.standard_normal(n) * np.exp2(rng.integers(-20, 126, n))).astype(np.float32)
    S[:4] = [0.0, -0.0, 3.0, -5.0]
    inv[:4] = [7.0, np.inf, 0.0, np.inf]
    for k in (0, -1, -2, -7, -20):
        alpha = np.float32(2.0 ** k)
        a, b = _unfolded(S, inv, alpha), _folded(S, inv, alpha)
        aS = np.abs(S.astype(np.float64) * float(alpha))
        inside = (aS == 0) | (aS >= 2.0 ** -126)
        assert inside.mean() > 0.9
        assert _same(a, b)[inside].all(), k
        # signed zeros agree too (they decide floor(-0) = -0 against floor(+0))
        assert (np.signbit(a) == np.signbit(b))[inside & ~np.isnan(a)].all()


def test_alpha_fold_differs_by_less_than_two_to_minus_21_in_the_subnormal_range():
    rng = np.random.default_rng(29)
    n = 1_000_000
    alpha = np.float32(0.25)
    # |alpha S| below 2^-126: fl(alpha S) is rounded in the subnormal range
    S = (rng.uniform(-1, 1, n) * np.exp2(rng.integers(-150, -124, n))).astype(np.float32)
    inv = np.exp2(rng.uniform(0, 127.9, n)).astype(np.float32)
    a = _unfolded(S, inv, alpha).astype(np.float64)
    b = _folded(S, inv, alpha).astype(np.float64)
    fin = np.isfinite(a) & np.isfinite(b)
    assert fin.all()
    assert np.abs(a - b).max() < 2.0 ** -21
    assert (a != b).any(), "the subnormal range does round differently"
