"""CPU checks of the comparison rules the GPU parity tests apply (tests/parity.py): the rule
for N~ elements that round to the other bf16 neighbour must accept a flip that the R
difference explains and reject every other kind of difference."""
import numpy as np
import pytest

from oracle import qgalore_oracle as O
from tests import parity as PAR

F32 = np.float32


def _case(r=32, n=64, m=48, seed=0):
    rng = np.random.default_rng(seed)
    N_o = (rng.standard_normal((r, n)) * 1e-3).astype(F32)
    P = O.bf16_round(rng.standard_normal((m, r)).astype(F32) * 0.1)
    return N_o, P


def _midpoint_pair(x):
    """A value just below the bf16 midpoint above x and one just above it (fp32)."""
    lo = O.bf16_round(np.array([x], F32))[0]
    hi = np.nextafter(lo, F32(np.inf) if lo >= 0 else F32(-np.inf), dtype=F32)
    for _ in range(1 << 16):            # the next bf16 value away from zero
        if O.bf16_round(np.array([hi], F32))[0] != lo:
            break
        hi = np.nextafter(hi, F32(np.inf) if lo >= 0 else F32(-np.inf), dtype=F32)
    hi_b = O.bf16_round(np.array([hi], F32))[0]
    mid = (np.float64(lo) + np.float64(hi_b)) / 2
    below = F32(mid - abs(mid) * 2e-7)
    above = F32(mid + abs(mid) * 2e-7)
    return below, above


def test_no_flip_carries_nothing():
    N_o, P = _case()
    assert np.all(PAR.explained_n_flips(N_o, O.bf16_round(N_o), N_o, O.bf16_round(N_o), P,
                                        0.25) == 0)


def test_an_explained_flip_is_accepted_and_carried_in_its_column_only():
    N_o, P = _case()
    N_g = N_o.copy()
    below, above = _midpoint_pair(N_o[3, 7])
    N_o[3, 7], N_g[3, 7] = below, above
    Nb_o, Nb_g = O.bf16_round(N_o), O.bf16_round(N_g)
    assert Nb_o[3, 7] != Nb_g[3, 7]
    carried = PAR.explained_n_flips(N_g, Nb_g, N_o, Nb_o, P, 0.25)
    assert carried.shape == (P.shape[0], N_o.shape[1])
    assert np.all(carried[:, 7] > 0)
    assert not np.any(np.delete(carried, 7, axis=1))
    d = abs(float(Nb_g[3, 7]) - float(Nb_o[3, 7]))
    assert np.allclose(carried[:, 7], 0.25 * np.abs(P[:, 3]) * d)


def test_a_steep_flip_across_several_values_is_accepted():
    """At t = 1, N = -lr R / (|R| + eps) is steep where R is near zero: a small R difference
    moves N across several bf16 values. The flip is explained when N itself moved that far."""
    N_o, P = _case()
    N_g = N_o.copy()
    N_o[4, 6] = F32(1.0e-4)
    N_g[4, 6] = F32(1.7e-4)               # many bf16 values away
    Nb_o, Nb_g = O.bf16_round(N_o), O.bf16_round(N_g)
    carried = PAR.explained_n_flips(N_g, Nb_g, N_o, Nb_o, P, 0.25)
    d = abs(float(Nb_g[4, 6]) - float(Nb_o[4, 6]))
    assert np.allclose(carried[:, 6], 0.25 * np.abs(P[:, 4]) * d)


def test_a_gpu_update_that_is_not_the_rounding_of_its_n_is_rejected():
    N_o, P = _case()
    Nb_o = O.bf16_round(N_o)
    Nb_g = Nb_o.copy()
    Nb_g.view(np.uint32)[2, 2] += 2 << 16
    with pytest.raises(AssertionError, match="not bf16"):
        PAR.explained_n_flips(N_o, Nb_g, N_o, Nb_o, P, 0.25)


def test_an_oracle_update_that_is_not_the_rounding_of_its_n_is_rejected():
    N_o, P = _case()
    Nb_o = O.bf16_round(N_o)
    Nb_bad = Nb_o.copy()
    Nb_bad.view(np.uint32)[5, 9] += 1 << 16
    with pytest.raises(AssertionError, match="not bf16"):
        PAR.explained_n_flips(N_o, Nb_o, N_o, Nb_bad, P, 0.25)


def _flips_at_midpoints(count, r=64, n=256):
    N_o, P = _case(r=r, n=n)
    N_g = N_o.copy()
    for k in range(count):
        i, j = k % r, (7 * k) % n
        below, above = _midpoint_pair(N_o[i, j])
        N_o[i, j], N_g[i, j] = below, above
    return N_g, N_o, P


def test_expected_flips_follow_the_n_difference():
    """E counts min(1, delta / u): a difference of a quarter of the bf16 spacing at every
    element expects a quarter of the elements to flip, and that many are accepted."""
    rng = np.random.default_rng(3)
    N_o = O.bf16_round((rng.standard_normal((64, 256)) * 1e-3).astype(F32))
    u = PAR._bf16_spacing(N_o)
    shift = rng.uniform(-0.5, 0.5, N_o.shape) * u      # positions inside each bf16 cell
    N_o = (N_o + shift).astype(F32)
    N_g = (N_o + 0.25 * u).astype(F32)
    E = PAR.expected_n_flips(N_g, N_o)
    assert abs(E / N_o.size - 0.25) < 0.01
    flips = int((O.bf16_round(N_g) != O.bf16_round(N_o)).sum())
    assert abs(flips - E) < 5 * np.sqrt(E)
    P = _case(r=64, n=256)[1]
    PAR.explained_n_flips(N_g, O.bf16_round(N_g), N_o, O.bf16_round(N_o), P, 0.25)


def test_a_few_explained_flips_are_accepted():
    N_g, N_o, P = _flips_at_midpoints(3)
    PAR.explained_n_flips(N_g, O.bf16_round(N_g), N_o, O.bf16_round(N_o), P, 0.25)


def test_more_flips_than_the_n_difference_explains_are_rejected():
    """Ten flips, each next to a midpoint, with differences of 4e-7 of N: the differences
    expect about 1e-3 flips in all, so ten point to misplaced boundaries."""
    N_g, N_o, P = _flips_at_midpoints(10)
    assert PAR.expected_n_flips(N_g, N_o) < 0.01
    with pytest.raises(AssertionError, match="another bf16 value"):
        PAR.explained_n_flips(N_g, O.bf16_round(N_g), N_o, O.bf16_round(N_o), P, 0.25)


def test_fp32_accumulation_rule():
    rng = np.random.default_rng(4)
    ref = rng.standard_normal((32, 64))
    PAR.assert_fp32_accumulation(ref * (1 + 1e-6 * rng.standard_normal(ref.shape)), ref, "R")
    low = O.bf16_round(ref.astype(F32))             # one bf16 rounding of every element
    with pytest.raises(AssertionError, match="rms difference"):
        PAR.assert_fp32_accumulation(low, ref, "R")
