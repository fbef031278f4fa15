"""Pins for the oracle's zero-point search (CPU only).

The variant keeps the full method's scale (the zero-aware quantizer of the
Echo paper card's Table 8: range widened to contain 0, binary16 scale) and
searches the integer zero point: z in [0, Qm] minimizing the group's squared
error measured in units of the scale on the fp32 products t_i = v_i * (1/s)
that pick the codes, E(z) = sum_i (clamp(rint(t_i) + z, 0, Qm) - z - t_i)^2,
the smallest z on ties.  The oracle evaluates a z-independent shift of E in
double; these pins recompute E itself for every z with exact rationals.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle


def f16(bits: int) -> float:
    return float(np.array([bits], np.uint16).view(np.float16)[0])


def nearest_even(t: Fr) -> int:
    fl = t.numerator // t.denominator
    d = t - fl
    if d < Fr(1, 2):
        return fl
    if d > Fr(1, 2):
        return fl + 1
    return fl if fl % 2 == 0 else fl + 1


def products(v32, sh):
    """t_i = v_i * (1/s) as the fp32 operations give them, as exact rationals."""
    s = np.float32(f16(sh))
    inv = np.float32(1.0) / s
    return [Fr(float(np.float32(x) * inv)) for x in v32]


def sq_error(t, z, Qm):
    return sum((min(max(nearest_even(ti) + z, 0), Qm) - z - ti) ** 2 for ti in t)


def check_group(v32, bits):
    Qm = (1 << bits) - 1
    q, sh, zh = oracle.quantize_group(v32, bits, "mse")
    q0, sh0, zh0 = oracle.quantize_group(v32, bits)
    assert sh == sh0                                      # the full method's scale
    if sh == 0:
        assert zh == 0 and not q.any()
        return None
    t = products(v32, sh)
    errs = [sq_error(t, z, Qm) for z in range(Qm + 1)]
    best = min(errs)
    z_star = errs.index(best)                             # smallest minimizer
    z = f16(zh)
    assert z == z_star, (v32, z, z_star)
    assert q.tolist() == [min(max(nearest_even(ti) + z_star, 0), Qm) for ti in t]
    # never worse than the closed-form zero point of the full method
    assert best <= errs[int(f16(zh0))]
    # the squared error is convex in z (second differences >= 0)
    assert all(errs[k - 1] - 2 * errs[k] + errs[k + 1] >= 0 for k in range(1, Qm))
    return z_star, int(f16(zh0))


@pytest.mark.parametrize("bits", [4, 8])
def test_exhaustive_exact_search_on_tiny_groups(bits):
    """Every z of every group, exact: one-decimal groups (the shape of Fig. 4's
    example), random magnitudes, one-sided groups and exact ties."""
    rng = np.random.default_rng(70 + bits)
    moved = 0
    trials = 1500 if bits == 4 else 250
    for trial in range(trials):
        g = int(rng.choice([2, 3, 4, 6, 8]))
        kind = trial % 4
        if kind == 0:
            v = rng.integers(-40, 41, size=g) / 10
        elif kind == 1:
            v = rng.standard_normal(g) * 10.0 ** rng.uniform(-6, 3)
        elif kind == 2:
            v = np.abs(rng.standard_normal(g)) * (1 if trial % 8 < 4 else -1)
        else:
            v = (rng.integers(-30, 31, size=g) + 0.5) * 2.0 ** -4   # exact half-code products
        r = check_group(v.astype(np.float32), bits)
        if r is not None and r[0] != r[1]:
            moved += 1
    assert moved > 0                                      # the search does move some zero points


def test_hand_worked_group_where_the_search_wins():
    """[-1.3, -1.0, 1.7, 0.0], b = 4.  Range 3.0, 3.0/15 = 0.2 rounds down to
    binary16 1638/8192 = 0.199951171875 (bits 0x3266), so 1/s = 5.0012...
    and t = v/s = -6.5016, -5.0012, 8.5021, 0: the rounded codes span -7 .. 9,
    17 levels for 16 codes.  The full method's zero point rint(6.5016) = 7
    clamps the top value to code 15 (decoded 8 s, error 0.5021 in units of s);
    z = 6 instead clamps the bottom value to code 0 (decoded -6 s, error
    0.4984) and represents 1.7 as 9 s (error 0.4979).  Squared error over the
    group: 0.5005 at z = 7, 0.4995 at z = 6; the search takes z = 6 (bits
    0x4600), codes 0, 1, 15, 6 against the full method's 0, 2, 15, 7."""
    v = np.array([-1.3, -1.0, 1.7, 0.0], np.float32)
    q, sh, zh = oracle.quantize_group(v, 4, "mse")
    q0, sh0, zh0 = oracle.quantize_group(v, 4)
    assert (sh, sh0) == (0x3266, 0x3266)
    assert (zh0, zh) == (0x4700, 0x4600)
    assert q0.tolist() == [0, 2, 15, 7] and q.tolist() == [0, 1, 15, 6]
    t = products(v, sh)
    assert sq_error(t, 6, 15) < sq_error(t, 7, 15)


def test_hand_worked_tie_takes_the_smaller_zero_point():
    """[-3.5, 11.5, 4.5, 5.5, -2.5, 0.5, 6.5, -0.5] * 2^-4: s = 2^-4 exactly and
    every t is a half-integer.  At z = 4 (the full method) the top value's
    code 12 + 4 clamps to 15 (error 0.5); at z = 3 the bottom value's -4 + 3
    clamps to 0 (error 0.5) instead: equal squared errors, so the search
    takes the smaller zero point, z = 3, codes 0, 15, 7, 9, 1, 3, 9, 3."""
    v = (np.array([-3.5, 11.5, 4.5, 5.5, -2.5, 0.5, 6.5, -0.5]) * 2.0 ** -4).astype(np.float32)
    q, sh, zh = oracle.quantize_group(v, 4, "mse")
    assert (sh, zh) == (0x2C00, 0x4200)
    assert q.tolist() == [0, 15, 7, 9, 1, 3, 9, 3]


@pytest.mark.parametrize("bits", [4, 8])
def test_full_groups_never_worse_than_the_closed_form(bits):
    """128-element groups of the workloads' distributions: the searched zero
    point's exact squared error is at most the full method's, and equal to
    it when nothing is clamped at the closed-form zero point."""
    Qm = (1 << bits) - 1
    rng = np.random.default_rng(90 + bits)
    for trial in range(60):
        kind = trial % 3
        if kind == 0:
            v = rng.laplace(size=128)
        elif kind == 1:
            v = rng.standard_normal(128)
            v[rng.integers(0, 128, 2)] *= 20
        else:
            v = rng.standard_normal(128) * 0.05 + rng.uniform(-0.1, 0.1)
        v = v.astype(np.float32)
        q, sh, zh = oracle.quantize_group(v, bits, "mse")
        q0, sh0, zh0 = oracle.quantize_group(v, bits)
        t = products(v, sh)
        e, e0 = sq_error(t, int(f16(zh)), Qm), sq_error(t, int(f16(zh0)), Qm)
        assert e <= e0
        if zh != zh0:
            assert e < e0 or int(f16(zh)) < int(f16(zh0))


def test_all_zero_group():
    for v in ([0.0, 0.0], [-0.0, 0.0, 0.0, -0.0]):
        q, sh, zh = oracle.quantize_group(np.array(v, np.float32), 4, "mse")
        assert sh == 0 and zh == 0 and not q.any()
