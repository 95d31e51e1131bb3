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
