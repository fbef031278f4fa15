"""Pins for the oracle's two ablation quantizers of the Echo paper card's
Table 8, "naive zero-point" and "symmetric grid" (CPU only).  The pages name
them and rank them below the zero-aware asymmetric quantizer, but print no
formula; the readings are:

  naive      the min/max affine quantizer with a real-valued zero point:
             range [min v, max v] (not widened to 0), s = binary16((hi-lo)/Qm),
             z = binary16(-lo/s), q = clamp(round(v/s + z), 0, Qm);
  symmetric  a grid symmetric about 0: s = binary16(max|v| / (2^(b-1) - 1)),
             z = 2^(b-1), q = clamp(round(v/s) + z, 0, Qm).

Both keep the full method's parameter word (binary16 s, binary16 z) and its
decode v_hat = (q - z) * s.  Pins: exact-rational choice of s (and z), brute
force over every code, grid round-trips, zero-awareness of the symmetric grid
and its absence in the naive quantizer, and the decode's single rounding.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from test_oracle_quantizer import brute_code, f16_value, nearest_f16_candidates

def brute_code_wide(target: Fr, Qm: int, window: Fr):
    dists = [abs(target - q) for q in range(Qm + 1)]
    best = min(dists)
    ok = {q for q in range(Qm + 1) if dists[q] == best}
    fl = target.numerator // target.denominator
    if abs(target - fl - Fr(1, 2)) <= window:
        ok |= {min(max(fl, 0), Qm), min(max(fl + 1, 0), Qm)}
    return ok


def check_naive(v32, bits):
    Qm = (1 << bits) - 1
    q, sh, zh = oracle.quantize_group(v32, bits, "naive")
    vals = [Fr(float(t)) for t in v32]
    lo, hi = min(vals), max(vals)
    if hi == lo:
        assert sh == 0 and zh == 0 and not q.any()
        return
    assert sh in nearest_f16_candidates((hi - lo) / Qm), (v32, hex(sh))
    s = f16_value(sh)
    zr = -lo / s
    # z: binary16 of -lo/s (two fp32 roundings before it)
    z = f16_value(zh & 0x7FFF) * (-1 if zh & 0x8000 else 1)
    if abs(zr) < 65504:
        assert abs(z - zr) <= abs(zr) * Fr(1, 1 << 10) + Fr(1, 1 << 24), (v32, float(z), float(zr))
    for i, vi in enumerate(vals):
        target = vi / s + z
        window = Fr(1, 1 << 20) * (abs(vi / s) + abs(z) + 1)
        assert int(q[i]) in brute_code_wide(target, Qm, window), (v32, i, int(q[i]), float(target))
        d = Fr(oracle.dequant(int(q[i]), sh, zh))
        exact = (int(q[i]) - z) * s
        # q - z rounds to fp32 when z has bits below q's last place, then the
        # product rounds: at most two roundings of half an ulp each
        assert abs(d - exact) <= abs(exact) * Fr(1, 1 << 23), (v32, i)


def check_symmetric(v32, bits):
    Qm, Qh, mid = (1 << bits) - 1, (1 << (bits - 1)) - 1, 1 << (bits - 1)
    q, sh, zh = oracle.quantize_group(v32, bits, "symmetric")
    assert f16_value(zh) == mid
    vals = [Fr(float(t)) for t in v32]
    a = max(abs(t) for t in vals)
    if a == 0:
        assert sh == 0 and np.all(q == mid)
        return
    assert sh in nearest_f16_candidates(a / Qh), (v32, hex(sh))
    s = f16_value(sh)
    for i, vi in enumerate(vals):
        assert int(q[i]) in brute_code(vi / s + mid, Qm), (v32, i, int(q[i]))
        assert Fr(oracle.dequant(int(q[i]), sh, zh)) == (int(q[i]) - mid) * s    # exact


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("quant", ["naive", "symmetric"])
def test_brute_force_one_decimal_lattice(bits, quant):
    lattice = np.array([k / 10 for k in range(-30, 31)], dtype=np.float32)
    check = check_naive if quant == "naive" else check_symmetric
    for a in lattice:
        for b in lattice[::3]:
            check(np.array([a, b], dtype=np.float32), bits)
    rng = np.random.default_rng(60 + bits)
    for _ in range(400):
        check(rng.choice(lattice, size=4).astype(np.float32), bits)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("quant", ["naive", "symmetric"])
def test_brute_force_random_magnitudes(bits, quant):
    rng = np.random.default_rng(70 + bits)
    check = check_naive if quant == "naive" else check_symmetric
    for trial in range(600):
        g = int(rng.choice([2, 4, 8]))
        v = (rng.standard_normal(g) * 10.0 ** rng.uniform(-4, 3)).astype(np.float32)
        if trial % 5 == 0:
            v = (np.abs(v) + 10.0 ** rng.uniform(-2, 1)).astype(np.float32)   # one-sided, away from 0
        check(v, bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_symmetric_round_trip_and_zero(bits):
    """Values (k - mid) * s with both ends of the symmetric range present come
    back exactly; 0 is the middle code and decodes to +0."""
    Qm, Qh, mid = (1 << bits) - 1, (1 << (bits - 1)) - 1, 1 << (bits - 1)
    rng = np.random.default_rng(80 + bits)
    for _ in range(2000):
        sh = int(rng.integers(0x0400, 0x5800))
        s = np.array([sh], np.uint16).view(np.float16).astype(np.float32)[0]
        g = int(rng.choice([4, 16, 128]))
        k = rng.integers(mid - Qh, mid + Qh + 1, size=g)
        k[0] = mid + Qh if rng.random() < 0.5 else mid - Qh
        k[1] = mid
        v = ((k - mid).astype(np.float32) * s).astype(np.float32)
        q, sh2, zh = oracle.quantize_group(v, bits, "symmetric")
        assert sh2 == sh and np.array_equal(q, k.astype(np.uint8))
        assert oracle.dequant(int(q[1]), sh2, zh) == 0.0


@pytest.mark.parametrize("bits", [4, 8])
def test_naive_round_trip_and_missing_zero(bits):
    """Values (k - z) * s with z a binary16 value of few fraction bits and
    codes 0 and Qm present come back exactly; and, unlike the zero-aware
    quantizer, an exact 0 in a group generally does not decode to 0."""
    Qm = (1 << bits) - 1
    rng = np.random.default_rng(90 + bits)
    for _ in range(2000):
        sh = int(rng.integers(0x2000, 0x5000))
        s = np.array([sh], np.uint16).view(np.float16).astype(np.float32)[0]
        z = np.float32(rng.integers(-400, 400) / 4.0)         # quarter steps: exact products
        g = int(rng.choice([4, 16, 128]))
        k = rng.integers(0, Qm + 1, size=g)
        k[0], k[1] = 0, Qm
        v = ((k.astype(np.float32) - z) * s).astype(np.float32)
        exact = [(Fr(int(a)) - Fr(float(z))) * Fr(float(s)) for a in k]
        if any(Fr(float(a)) != b for a, b in zip(v, exact)):
            continue
        q, sh2, zh = oracle.quantize_group(v, bits, "naive")
        assert sh2 == sh, (hex(sh), hex(sh2))
        assert f16_value(zh & 0x7FFF) * (-1 if zh & 0x8000 else 1) == Fr(float(z))
        assert np.array_equal(q, k.astype(np.uint8))
    # the missing zero: a group whose range excludes 0, or whose zero point is fractional
    misses = 0
    for _ in range(200):
        v = (rng.standard_normal(128) + rng.uniform(-1, 1)).astype(np.float32)
        v[5] = 0.0
        q, sh, zh = oracle.quantize_group(v, bits, "naive")
        misses += oracle.dequant(int(q[5]), sh, zh) != 0.0
        qz, shz, zhz = oracle.quantize_group(v, bits)
        assert oracle.dequant(int(qz[5]), shz, zhz) == 0.0            # zero-aware keeps it
    assert misses > 150


@pytest.mark.parametrize("quant", ["naive", "symmetric", "mse"])
@pytest.mark.parametrize("P", [2, 4])
def test_call_structure_holds_for_every_quantizer(quant, P):
    """Identical outputs, at most two quantizations, and the error identity do
    not depend on which quantizer the call uses."""
    rng = np.random.default_rng(100 + P)
    n = P * 128 * 3
    xs = [oracle.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32)) for _ in range(P)]
    outs, qdepth, qwork = oracle.allreduce(xs, bits=4, quant=quant, want_counts=True)
    for r in range(1, P):
        assert outs[r].tobytes() == outs[0].tobytes()
    assert np.all(qdepth == 2) and np.all(qwork == n)
    comps = [np.zeros(n, np.float32) for _ in range(P)]
    errs = [np.zeros(n, np.float32) for _ in range(P)]
    outs, _, _ = oracle.allreduce(xs, bits=4, quant=quant, ef=True, comps=comps, errs=errs)
    xsum = sum((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for x in xs)
    esum = sum(e.astype(np.float64) for e in errs)
    mag = sum(np.abs((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)) for x in xs)
    assert np.all(np.abs(outs[0] - xsum - esum) <= (P + 2) * 2.0 ** -24 * (mag + np.abs(esum) + np.abs(outs[0])))


@pytest.mark.parametrize("bits", [4, 8])
def test_naive_zero_point_of_a_zero_minimum_is_plus_zero(bits):
    """When a group's minimum is a zero, the naive zero point is +0 whichever
    signed zero the minimum is and wherever it sits: the result does not
    depend on which of two equal minima a reduction keeps."""
    rng = np.random.default_rng(120 + bits)
    for _ in range(300):
        v = np.abs(rng.standard_normal(128)).astype(np.float32) + np.float32(0.01)
        k = rng.choice(128, size=3, replace=False)
        v[k[0]] = -0.0
        v[k[1]] = 0.0
        if rng.random() < 0.5:
            v[k[2]] = -0.0
        q, sh, zh = oracle.quantize_group(v, bits, "naive")
        assert zh == 0x0000, hex(zh)
        w = v.copy()
        w[k[0]], w[k[1]] = w[k[1]], w[k[0]]
        assert oracle.quantize_group(w, bits, "naive")[1:] == (sh, zh)
        assert oracle.dequant(int(q[k[0]]), sh, zh) == 0.0


def test_both_ablations_at_once_is_rejected():
    n, P = 4 * 128, 4
    x = np.zeros(n, np.uint16)
    for flags in (oracle.Q_NAIVE | oracle.Q_SYMMETRIC, oracle.Q_NAIVE | oracle.Q_MSE, oracle.Q_SYMMETRIC | oracle.Q_MSE):
        with pytest.raises(oracle.OracleError):
            oracle.quantize_ef(x, None, n, P, 0, 0, 128, 4, 128, np.zeros(n, np.uint8),
                               np.zeros(2 * n // 128, np.uint16), None, flags)


@pytest.mark.parametrize("quant", ["zero_aware", "naive", "symmetric", "mse"])
@pytest.mark.parametrize("bits", [4, 8])
def test_steps_use_the_selected_quantizer(quant, bits):
    """The flag bits reach the group quantizer pinned above: the push step's
    codes and parameters are that quantizer's, group by group, and a one-rank
    call is one round trip through it."""
    flag = oracle.QUANTS[quant]
    rng = np.random.default_rng(110 + bits)
    P, n, g = 4, 4 * 128 * 2, 128
    x = oracle.f32_to_bf16_bits((rng.standard_normal(n) + 0.7).astype(np.float32))
    v = (x.astype(np.uint32) << 16).view(np.float32)
    codes = np.zeros(oracle.code_bytes(n, bits), np.uint8)
    params = np.zeros(2 * n // g, np.uint16)
    oracle.quantize_ef(x, None, n, P, 0, 0, n // P, bits, g, codes, params, None, flag)
    for grp in range(n // P // g, n // g):                       # segments 1..3 (rank 0 pushes them)
        q, sh, zh = oracle.quantize_group(v[grp * g:(grp + 1) * g], bits, quant)
        assert (int(params[2 * grp]), int(params[2 * grp + 1])) == (sh, zh), (quant, grp)
        if bits == 8:
            assert np.array_equal(codes[grp * g:(grp + 1) * g], q)
        else:
            packed = codes[grp * g // 2:(grp + 1) * g // 2]
            assert np.array_equal(packed & 0x0F, q[0::2]) and np.array_equal(packed >> 4, q[1::2])
    outs, _, _ = oracle.allreduce([x[:256]], bits=bits, quant=quant)
    for grp in range(2):
        q, sh, zh = oracle.quantize_group(v[grp * g:(grp + 1) * g], bits, quant)
        want = np.array([oracle.dequant(int(c), sh, zh) for c in q], np.float32)
        assert np.array_equal(outs[0][grp * g:(grp + 1) * g], want)
