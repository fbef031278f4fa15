"""Hand-worked exact cases for the oracle (CPU only): rounding ties, the
packed code layout and the owner's summation order.

Sources: the Echo paper card (arXiv 2610.14277), Table 8 (zero-aware
asymmetric quantizer and its two ablations, g = 128), Fig. 2(a) (the owner
adds the decoded peer copies to its own copy in high precision); the
PhantomByte article, "The cancellation rule" (4-bit integer codes, binary16
parameters per group).  The pages fix neither the tie rule, nor the nibble
order, nor the order of the sum; the readings taken are:

  * ties: rint rounds half to even, for the codes of every quantizer and for
    the zero-aware zero point; the integer zero point is added after rounding,
    the naive (real) zero point before;
  * packing: for 4-bit codes element i sits in byte i/2, the low nibble when
    i is even;
  * the owner's sum: fp32, left to right in rank order j = 0..P-1, the owner's
    own (unquantized) term at position `owner`.

Every case below uses a power-of-two scale s, so 1/s is exact and every
v * (1/s) is exact: the value handed to the rounding step is an exact
half-integer and the two neighbours are equally near.  Expected values are
worked by hand (each docstring shows the arithmetic); a round-half-away rule
(roundf), a zero point added on the wrong side of the rounding, a swapped
nibble order or another summation order each changes at least one of them.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle

S = 2.0 ** -4          # scale used by the tie groups: binary16 0x2C00, 1/s = 16 exactly


def f16_bits(x: float) -> int:
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def group(mults, s=S):
    """fp32 group whose elements are the given multiples of s (all exact)."""
    v = np.array([m * s for m in mults], dtype=np.float32)
    assert all(Fr(float(a)) == Fr(m) * Fr(s) for a, m in zip(v, mults))
    return v


def test_zero_aware_4bit_tie_on_the_zero_point_and_codes():
    """Group [-2.5, 12.5, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5] * s, s = 2^-4.

    lo = -2.5 s, hi = 12.5 s, hi - lo = 15 s, (hi - lo)/15 = s = 0.0625 exactly
    -> scale bits 0x2C00, 1/s = 16.
    z = rint(-lo/s) = rint(2.5) = 2 (half to even; half away would give 3)
    -> zero bits 0x4000.
    codes q = rint(v/s) + 2:
      rint(-2.5) = -2 -> 0;  rint(12.5) = 12 -> 14;  rint(0.5) = 0 -> 2;
      rint(1.5) = 2 -> 4;    rint(2.5) = 2 -> 4;     rint(3.5) = 4 -> 6;
      rint(-0.5) = -0 -> 2;  rint(-1.5) = -2 -> 0.
    decoded (q - 2) * s: -0.125, 0.75, 0, 0.125, 0.125, 0.25, 0, -0.125."""
    v = group([-2.5, 12.5, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5])
    q, sh, zh = oracle.quantize_group(v, 4)
    assert (sh, zh) == (0x2C00, 0x4000), (hex(sh), hex(zh))
    assert q.tolist() == [0, 14, 2, 4, 4, 6, 2, 0]
    assert [oracle.dequant(int(a), sh, zh) for a in q] == [-0.125, 0.75, 0.0, 0.125, 0.125, 0.25, 0.0, -0.125]


def test_zero_aware_4bit_ties_with_an_odd_zero_point_neighbour():
    """Group [-3.5, 11.5, 4.5, 5.5, -2.5, 0.5, 6.5, -0.5] * s, s = 2^-4.

    hi - lo = 15 s -> s = 0.0625 (0x2C00); z = rint(3.5) = 4 (0x4400).
    codes q = clamp(rint(v/s) + 4, 0, 15):
      rint(-3.5) = -4 -> 0;  rint(11.5) = 12 -> 16, clamped to 15;
      rint(4.5) = 4 -> 8;    rint(5.5) = 6 -> 10;   rint(-2.5) = -2 -> 2;
      rint(0.5) = 0 -> 4;    rint(6.5) = 6 -> 10;   rint(-0.5) = -0 -> 4.
    (Half away from zero: 0, 15, 9, 10, 1, 5, 11, 3.)"""
    v = group([-3.5, 11.5, 4.5, 5.5, -2.5, 0.5, 6.5, -0.5])
    q, sh, zh = oracle.quantize_group(v, 4)
    assert (sh, zh) == (0x2C00, 0x4400), (hex(sh), hex(zh))
    assert q.tolist() == [0, 15, 8, 10, 2, 4, 10, 4]


def test_zero_aware_4bit_code_ties_with_an_odd_zero_point():
    """Group [-3, 12, 0.5, 1.5, -0.5, 2.5, -2.5, 6.5] * s, s = 2^-4.

    hi - lo = 15 s -> s = 0.0625 (0x2C00); z = rint(3) = 3 (0x4200), odd, so
    the integer zero point must be added after rounding:
    codes q = rint(v/s) + 3: 0, 15, 0 + 3 = 3, 2 + 3 = 5, -0 + 3 = 3,
    2 + 3 = 5, -2 + 3 = 1, 6 + 3 = 9.
    (Adding z before rounding gives rint(3.5) = 4, rint(4.5) = 4, rint(2.5) = 2,
    rint(5.5) = 6, rint(0.5) = 0, rint(9.5) = 10 instead.)"""
    v = group([-3, 12, 0.5, 1.5, -0.5, 2.5, -2.5, 6.5])
    q, sh, zh = oracle.quantize_group(v, 4)
    assert (sh, zh) == (0x2C00, 0x4200), (hex(sh), hex(zh))
    assert q.tolist() == [0, 15, 3, 5, 3, 5, 1, 9]


def test_zero_aware_8bit_ties():
    """Group [-100.5, 154.5, 0.5, 1.5, -0.5, 27.5, -27.5, 2.5] * s, s = 2^-4.

    hi - lo = 255 s, /255 = s (0x2C00); z = rint(100.5) = 100 (binary16
    0x5640).  codes q = rint(v/s) + 100:
      -100 -> 0; 154 -> 254; 0 -> 100; 2 -> 102; -0 -> 100; 28 -> 128;
      -28 -> 72; 2 -> 102."""
    v = group([-100.5, 154.5, 0.5, 1.5, -0.5, 27.5, -27.5, 2.5])
    q, sh, zh = oracle.quantize_group(v, 8)
    assert (sh, zh) == (0x2C00, 0x5640), (hex(sh), hex(zh))
    assert q.tolist() == [0, 254, 100, 102, 100, 128, 72, 102]


def test_naive_zero_point_ties():
    """Naive zero point (Table 8 ablation), b = 4:
    group [-2.25, 12.75, 0.25, 1.25, -1.75, 2.25, 8.25, -0.75] * s, s = 2^-4.

    lo = -2.25 s, hi = 12.75 s, (hi - lo)/15 = s (0x2C00), 1/s = 16.
    z = binary16((0 - lo)/s) = 2.25 exactly (0x4080).
    codes q = rint(v/s + 2.25), the real zero point added before rounding:
      rint(0) = 0; rint(15) = 15; rint(2.5) = 2; rint(3.5) = 4; rint(0.5) = 0;
      rint(4.5) = 4; rint(10.5) = 10; rint(1.5) = 2.
    (Half away from zero: 0, 15, 3, 4, 1, 5, 11, 2.)"""
    v = group([-2.25, 12.75, 0.25, 1.25, -1.75, 2.25, 8.25, -0.75])
    q, sh, zh = oracle.quantize_group(v, 4, "naive")
    assert (sh, zh) == (0x2C00, 0x4080), (hex(sh), hex(zh))
    assert q.tolist() == [0, 15, 2, 4, 0, 4, 10, 2]


def test_symmetric_grid_ties():
    """Symmetric grid (Table 8 ablation), b = 4:
    group [7, -2.5, -0.5, 0.5, 1.5, 2.5, 3.5, -6.5] * s, s = 2^-4.

    max|v| = 7 s, /7 = s (0x2C00); z = 8 (0x4800).
    codes q = rint(v/s) + 8: 15, 6, 8, 8, 10, 10, 12, 2.
    (Half away from zero: 15, 5, 7, 9, 10, 11, 12, 1.)"""
    v = group([7, -2.5, -0.5, 0.5, 1.5, 2.5, 3.5, -6.5])
    q, sh, zh = oracle.quantize_group(v, 4, "symmetric")
    assert (sh, zh) == (0x2C00, 0x4800), (hex(sh), hex(zh))
    assert q.tolist() == [15, 6, 8, 8, 10, 10, 12, 2]


def nearest_even(t: Fr) -> int:
    """The integer nearest to t, the even one of the two when t is halfway."""
    fl = t.numerator // t.denominator
    d = t - fl
    if d < Fr(1, 2):
        return fl
    if d > Fr(1, 2):
        return fl + 1
    return fl if fl % 2 == 0 else fl + 1


@pytest.mark.parametrize("bits", [4, 8])
def test_exact_ties_over_many_scales_and_zero_points(bits):
    """Zero-aware groups built so that -lo/s and every v/s are exact
    half-integers or integers (half the groups with an integer -lo/s, so z
    takes odd values too), with s = 2^k over binary16's subnormal and
    normal range: the zero point and every unclamped code are the even
    neighbour, in exact arithmetic."""
    Qm = (1 << bits) - 1
    rng = np.random.default_rng(60 + bits)
    for trial in range(400):
        k = int(rng.integers(-24, 8))                    # s = 2^-24 (subnormal) .. 2^7
        s = 2.0 ** k
        z0 = int(rng.integers(1, Qm))
        lo_m = -(z0 + 0.5) if trial % 2 else -float(z0)  # -lo/s a tie, or an integer (odd z too)
        hi_m = lo_m + Qm                                 # hi - lo = Qm * s: the scale is s exactly
        mults = [lo_m, hi_m] + [float(m) / 2 for m in rng.integers(int(2 * lo_m), int(2 * hi_m) + 1, size=30)]
        v = group(mults, s)
        q, sh, zh = oracle.quantize_group(v, bits)
        assert sh == f16_bits(s), (trial, hex(sh))
        z = nearest_even(Fr(-lo_m))
        assert Fr(float(np.array([zh], np.uint16).view(np.float16)[0])) == z
        for qi, m in zip(q.tolist(), mults):
            want = nearest_even(Fr(m)) + z
            assert qi == min(max(want, 0), Qm), (trial, m, qi, want)


def test_packed_nibbles_hold_the_even_element_low():
    """The push writes the tie group of the first test into the message's
    code array: codes 0, 14, 2, 4, 4, 6, 2, 0 pack as bytes 0xE0, 0x42, 0x64,
    0x02 (element 2k in the low nibble of byte k, 2k + 1 in the high one).
    P = 2 ranks, g = 8, rank 0 pushes segment 1."""
    v = group([-2.5, 12.5, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5])
    n, P, g = 16, 2, 8
    x = np.zeros(n, np.uint16)
    comp = np.zeros(n, np.float32)
    comp[8:] = v                                        # u = f32(0) + comp = v exactly
    codes = np.full(n // 2, 0xAA, np.uint8)
    params = np.full(2 * n // g, 0xBEEF, np.uint16)
    oracle.quantize_ef(x, comp, n, P, 0, 0, n // P, 4, g, codes, params, None)
    assert codes.tolist() == [0xAA] * 4 + [0xE0, 0x42, 0x64, 0x02]
    assert params.tolist() == [0xBEEF, 0xBEEF, 0x2C00, 0x4000]


def bf16(x: float) -> int:
    b = np.array([x], np.float32).view(np.uint32)[0]
    assert b & 0xFFFF == 0
    return int(b >> 16)


@pytest.mark.parametrize("owner, want_acc0", [(0, 1.0), (2, 1.0 + 2.0 ** -23)])
def test_owner_sum_in_rank_order(owner, want_acc0):
    """P = 3 ranks, one group of g = 8 per segment.  At element 0 of the owner's
    group the owner's own term is 1.0 and each peer's decoded term is 2^-24;
    element 1 sets the peers' range (15 * 2^-24: scale 2^-24, the smallest
    binary16, z = 0, so 2^-24 decodes exactly).

    In fp32, 1 + 2^-24 is a tie and rounds to 1; 2^-24 + 2^-24 = 2^-23 is
    exact.  Rank order j = 0, 1, 2:
      owner 0: (1 + 2^-24) + 2^-24 = 1
      owner 2: (2^-24 + 2^-24) + 1 = 1 + 2^-23
    The owner's group then has lo = 0, hi = acc0: s = binary16(acc0/15)
    = 1092 * 2^-14 (nearest to 1/15), code 15, decoded 15 s = 16380/16384,
    and the owner's error 15 s - acc0: -2^-12 for owner 0,
    -2^-12 - 2^-23 for owner 2 (both exact)."""
    P, g = 3, 8
    n = P * g
    tiny = 2.0 ** -24
    xs = [np.zeros(n, np.uint16) for _ in range(P)]
    for j in range(P):
        base = owner * g
        if j == owner:
            xs[j][base] = bf16(1.0)
        else:
            xs[j][base] = bf16(tiny)
            xs[j][base + 1] = bf16(15 * tiny)
    codes = [np.zeros(n // 2, np.uint8) for _ in range(P)]
    params = [np.zeros(2 * n // g, np.uint16) for _ in range(P)]
    for j in range(P):
        if j != owner:
            oracle.quantize_ef(xs[j], None, n, P, j, 0, g, 4, g, codes[j], params[j], None)
            assert params[j][2 * owner] == 0x0001 and params[j][2 * owner + 1] == 0
    sc = np.zeros(n // 2, np.uint8)
    sp = np.zeros(2 * n // g, np.uint16)
    err = np.zeros(n, np.float32)
    oracle.reduce_segment(xs[owner], None, codes, params, P, owner, n, 0, g, 4, g, sc, sp, err)
    s = 1092 * 2.0 ** -14
    assert sp[2 * owner] == f16_bits(s) and sp[2 * owner + 1] == 0
    assert float(err[owner * g]) == 15 * s - want_acc0
