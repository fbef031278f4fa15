"""Pins for the oracle's group quantizer Q_b and its dequantizer (CPU only).

The quantizer is the "zero-aware asymmetric" one of the Echo paper card
(Table 8, full method, g = 128; Eqn. (8), named in appendix Fig. 4 with b = 4),
with binary16 scale and zero point (PhantomByte article, "The cancellation
rule").  The pages print no formula, so the reading is: the min/max range is
widened to contain 0, s = binary16((hi - lo) / (2^b - 1)), an integer zero
point z = round(-lo / s) so that 0 is exactly code z, and codes
q = clamp(round(v / s) + z, 0, 2^b - 1).

What pins it here, without re-running its own formula:
  * exact-rational choice of the scale (nearest binary16 to the real quotient);
  * brute force over every code and every zero point in exact arithmetic;
  * the grid round-trip (values already on a grid come back unchanged);
  * zero-awareness (0 -> code z -> exactly 0);
  * the element error bound derived from the definition;
  * three groups worked by hand (below).
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle

F16_POS_BITS = np.arange(1, 0x7C00, dtype=np.uint16)
F16_POS_VALS = F16_POS_BITS.view(np.float16).astype(np.float64)   # increasing, exact in float64


def f16_value(bits: int) -> Fr:
    return Fr(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def nearest_f16_candidates(r: Fr):
    """binary16 bit patterns a correct scale choice may return for the exact
    real quotient r > 0.  Normally exactly one (nearest, ties to even); both
    neighbours when r lies within 2^-22 (relative) of their midpoint, where the
    two fp32 roundings before the binary16 rounding may decide."""
    x = float(r)
    i = int(np.searchsorted(F16_POS_VALS, x))
    if i == 0:
        # below the smallest subnormal 2^-24: zero unless past the midpoint 2^-25
        lo_bits, hi_bits = None, int(F16_POS_BITS[0])
        lo_val, hi_val = Fr(0), f16_value(hi_bits)
    elif i >= F16_POS_VALS.size:
        return {0x7BFF}                         # above 65504: overflow, clamped to 65504
    else:
        lo_bits, hi_bits = int(F16_POS_BITS[i - 1]), int(F16_POS_BITS[i])
        lo_val, hi_val = f16_value(lo_bits), f16_value(hi_bits)
        if Fr(x) == hi_val and r == hi_val:
            return {hi_bits}
    mid = (lo_val + hi_val) / 2
    clamp0 = lambda b: 0x0001 if b is None else b   # zero scale -> 2^-24
    if abs(r - mid) <= mid * Fr(1, 1 << 22):
        return {clamp0(lo_bits), hi_bits}
    if r < mid:
        return {clamp0(lo_bits)}
    if r > mid:
        return {hi_bits}
    even = lo_bits if (lo_bits or 0) % 2 == 0 else hi_bits
    return {clamp0(even)}


def brute_code(target: Fr, Qm: int):
    """All codes in [0, Qm] at minimal distance from `target`, plus their
    neighbours when target is within 2^-14 of a half-integer (the fp32
    product v * (1/s) may round across it)."""
    dists = [abs(target - q) for q in range(Qm + 1)]
    best = min(dists)
    ok = {q for q in range(Qm + 1) if dists[q] == best}
    frac = target - (target.numerator // target.denominator)
    if abs(frac - Fr(1, 2)) <= Fr(1, 1 << 14):
        fl = target.numerator // target.denominator
        ok |= {min(max(fl, 0), Qm), min(max(fl + 1, 0), Qm)}
    return ok


def check_group_brute_force(v32: np.ndarray, bits: int):
    Qm = (1 << bits) - 1
    q, sh, zh = oracle.quantize_group(v32, bits)
    vals = [Fr(float(t)) for t in v32]
    lo = min([Fr(0)] + vals)
    hi = max([Fr(0)] + vals)
    if hi == lo:
        assert sh == 0 and zh == 0 and not q.any()
        return
    # scale: nearest binary16 to the exact (hi - lo) / Qm
    assert sh in nearest_f16_candidates((hi - lo) / Qm), (v32, hex(sh))
    s = f16_value(sh)
    # zero point: the integer in [0, Qm] nearest to -lo / s
    z = int(f16_value(zh))
    assert f16_value(zh) == z
    assert z in brute_code(-lo / s, Qm), (v32, z)
    # codes: for every element, the code in [0, Qm] whose grid value (q - z) * s
    # is nearest to v -- searched over all 2^b codes
    for i, vi in enumerate(vals):
        assert int(q[i]) in brute_code(vi / s + z, Qm), (v32, i, int(q[i]), z, float(s))
        # the dequantizer is exact: (q - z) * s with no rounding
        assert Fr(oracle.dequant(int(q[i]), sh, zh)) == (int(q[i]) - z) * s


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("g", [2, 4])
def test_brute_force_one_decimal_lattice(bits, g):
    """Fig. 4's example quantizes two-element groups of one-decimal values;
    sweep such groups (values k/10, |k| <= 30) exhaustively for g = 2 and at
    random for g = 4."""
    lattice = np.array([k / 10 for k in range(-30, 31)], dtype=np.float32)
    if g == 2:
        groups = [np.array([a, b], dtype=np.float32) for a in lattice for b in lattice[::3]]
    else:
        rng = np.random.default_rng(10 + bits)
        groups = [rng.choice(lattice, size=g).astype(np.float32) for _ in range(600)]
    for v in groups:
        check_group_brute_force(v, bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_brute_force_random_magnitudes(bits):
    rng = np.random.default_rng(20 + bits)
    for trial in range(800):
        g = int(rng.choice([2, 4, 8]))
        scale = 10.0 ** rng.uniform(-9, 5)          # down into binary16 subnormal scales
        v = (rng.standard_normal(g) * scale).astype(np.float32)
        if trial % 7 == 0:
            v = np.abs(v)                            # one-sided groups: z == 0
        if trial % 11 == 0:
            v = -np.abs(v)                           # z == Qm
        check_group_brute_force(v, bits)


def test_scale_clamps_and_all_zero_group():
    # all-zero group (including negative zero): scale +0, zero point 0, codes 0
    for v in ([0.0, 0.0], [-0.0, 0.0], [-0.0, -0.0, 0.0, 0.0]):
        q, sh, zh = oracle.quantize_group(np.array(v, dtype=np.float32), 4)
        assert sh == 0 and zh == 0 and not q.any()
    # a range so small that binary16 rounds the scale to zero -> 2^-24
    q, sh, zh = oracle.quantize_group(np.array([0.0, 1e-9], dtype=np.float32), 4)
    assert sh == 0x0001
    # a range so large that the scale overflows binary16 -> 65504
    q, sh, zh = oracle.quantize_group(np.array([-1e7, 1e7], dtype=np.float32), 4)
    assert sh == 0x7BFF


@pytest.mark.parametrize("bits", [4, 8])
def test_grid_round_trip(bits):
    """Values v_i = (k_i - z) * s with s a binary16 value and codes 0 and Qm
    both present come back with the same codes, scale and zero point: the
    range is exactly Qm * s, so the scale is recovered exactly, and each
    v_i * (1/s) lies within 2^-23 * 255 of an integer."""
    Qm = (1 << bits) - 1
    rng = np.random.default_rng(30 + bits)
    for trial in range(3000):
        if trial % 10 == 0:
            sh = int(rng.integers(1, 0x0400))               # subnormal binary16 scales
        else:
            sh = int(rng.integers(0x0400, 0x5C00))          # normal, up to 2^8
        s = np.array([sh], dtype=np.uint16).view(np.float16).astype(np.float32)[0]
        z = int(rng.integers(0, Qm + 1))
        g = int(rng.choice([2, 4, 16, 128]))
        k = rng.integers(0, Qm + 1, size=g)
        i0, i1 = rng.choice(g, size=2, replace=False)
        k[i0], k[i1] = 0, Qm
        v = ((k - z).astype(np.float32) * s).astype(np.float32)
        # exactness of the constructed values
        assert all(Fr(float(a)) == (int(b) - z) * Fr(float(s)) for a, b in zip(v, k))
        q, sh2, zh = oracle.quantize_group(v, bits)
        assert sh2 == sh, (hex(sh), hex(sh2), z, k)
        assert int(f16_value(zh)) == z and zh == int(np.array([z], np.float16).view(np.uint16)[0])
        assert np.array_equal(q, k.astype(np.uint8))


@pytest.mark.parametrize("bits", [4, 8])
def test_zero_awareness(bits):
    """Table 8's full method is zero-aware: an exact 0 maps to the zero-point
    code and decodes to exactly +0 -- for every zero point the quantizer picks."""
    Qm = (1 << bits) - 1
    rng = np.random.default_rng(40 + bits)
    seen = set()
    for trial in range(4000):
        g = 128
        v = (rng.standard_normal(g) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        shift = rng.uniform(-1.2, 1.2) * np.abs(v).max()
        v = (v + shift).astype(np.float32)
        zpos = rng.choice(g, size=8, replace=False)
        v[zpos] = 0.0
        q, sh, zh = oracle.quantize_group(v, bits)
        z = int(f16_value(zh))
        seen.add(z)
        assert np.all(q[zpos] == z)
        for i in zpos:
            d = oracle.dequant(int(q[i]), sh, zh)
            assert d == 0.0 and np.signbit(np.float32(d)) == False
    assert len(seen) >= min(Qm + 1, 200), len(seen)     # the sweep hit (nearly) every zero point


@pytest.mark.parametrize("bits", [4, 8])
def test_element_error_bound(bits):
    """From the definition: an element not clamped has |v - v_hat| <= s/2 +
    2^-22 |v| (rounding to the grid plus the two fp32 roundings of v * (1/s));
    clamping happens only at the range ends, where binary16 rounding of the
    scale can shrink the covered range by Qm * 2^-11 steps."""
    Qm = (1 << bits) - 1
    rng = np.random.default_rng(50 + bits)
    for trial in range(1500):
        kind = trial % 4
        if kind == 0:
            v = rng.standard_normal(128)
        elif kind == 1:
            v = rng.laplace(size=128)
        elif kind == 2:
            v = rng.standard_normal(128)
            v[rng.integers(0, 128, size=2)] *= 20.0
        else:
            v = rng.standard_normal(128) * 1e-3 + rng.uniform(-1, 1) * 1e-2
        v = (v * 10.0 ** rng.uniform(-2, 2)).astype(np.float32)
        q, sh, zh = oracle.quantize_group(v, bits)
        s = float(f16_value(sh))
        if sh < 0x0400 or sh == 0x7BFF:
            continue                                  # subnormal or clamped scale: excluded
        z = int(f16_value(zh))
        vhat = (q.astype(np.float64) - z) * s
        err = np.abs(v.astype(np.float64) - vhat)
        clamped = (q == 0) | (q == Qm)
        free = ~clamped
        assert np.all(err[free] <= s / 2 + 2.0 ** -22 * np.abs(v[free])), trial
        bound_all = s * (0.5 + 1.001 * Qm * 2.0 ** -11) + 2.0 ** -21 * np.abs(v).max()
        assert np.all(err <= bound_all), trial


def test_hand_worked_groups():
    """Three b = 4 groups worked by hand from the reading above.

    [-0.5, 1.0]: range 1.5, 1.5/15 = 0.1 -> binary16 1638/16384 = 0.0999755859375
      (bits 0x2E66); -lo/s = 5.0012... -> z = 5 (bits 0x4500); codes 0 and 15;
      decoded -5*s = -0.4998779296875 and 10*s = 0.999755859375.
    [0.0, 0.3]: lo = 0 -> z = 0; 0.3/15 = 0.02 -> binary16 1311/65536
      (bits 0x251F); 0.3/s = 14.9968 -> code 15, decoded 0.3000640869140625.
    [-0.4, -0.1]: hi = 0; 0.4/15 = 0.02667 -> binary16 1748/65536 = 437/16384
      (bits 0x26D4); z = round(14.9968) = 15 (bits 0x4B80); -0.1/s = -3.749 ->
      -4 + 15 = code 11, decoded -4*s = -0.106689453125.
    """
    cases = [
        ([-0.5, 1.0], 0x2E66, 0x4500, [0, 15], [-0.4998779296875, 0.999755859375]),
        ([0.0, 0.3], 0x251F, 0x0000, [0, 15], [0.0, 0.3000640869140625]),
        ([-0.4, -0.1], 0x26D4, 0x4B80, [0, 11], [-0.40008544921875, -0.106689453125]),
    ]
    for v, sh_w, zh_w, q_w, d_w in cases:
        q, sh, zh = oracle.quantize_group(np.array(v, dtype=np.float32), 4)
        assert (sh, zh) == (sh_w, zh_w), (v, hex(sh), hex(zh))
        assert list(q) == q_w
        assert [oracle.dequant(int(a), sh, zh) for a in q] == d_w
