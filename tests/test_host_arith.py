"""Host checks of arithmetic identities the HIP kernels rely on (CPU only).

The quantizers' scale is s32 = x / Q for a constant Q (2^b - 1 for the
zero-aware and naive quantizers, 2^(b-1) - 1 for the symmetric grid).  The
kernels compute it without a division, as q0 = x * RN(1/Q), r = fma(-q0, Q, x),
q = fma(r, RN(1/Q), q0).  tests/c/div_by_const_check.c checks, over every
finite fp32 x >= 0, that q is the IEEE quotient for Q = 15, 255, 7 and 127,
and that the plain product q0 is not (so the check can tell them apart).

Their reciprocal 1/s of a binary16 scale s is one Newton step from the
hardware reciprocal, r1 = fma(r0, fma(-s, r0, 1), r0).
tests/c/recip_scale_newton.c checks, for every positive finite binary16 s and
every r0 within two ulps of RN(1/s), that r1 is the IEEE quotient 1/s, and
that the same step misses it for some full 24-bit divisors (the 11-bit
significand is what makes it exact).  tests/test_gpu_recip_scale.py checks
the kernels' own function on the GPU for every binary16 scale.

The owner reduce decodes a peer's codes for an integer zero point as
fma(binary16(1024 + q), s, fma(-(1024 + z), s, 0)).
tests/c/biased_decode_check.c checks that this equals the two-step decode
(q - z) * s bit for bit for every positive finite binary16 s and every q, z
in [0, 255] (and s = 0 where q == z), and that a decode with two roundings
does differ at full 24-bit scales.

Where a quantizer's range holds 0, the group min/max reduce raw fp32 bit
patterns (unsigned for lo <= 0, signed for hi >= 0);
test_raw_bit_order_of_ranges_that_hold_zero checks that ordering.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_free_quotient_is_exact_for_every_input(tmp_path):
    exe = tmp_path / "div_by_const_check"
    subprocess.run(["gcc", "-O3", "-march=native", "-fopenmp", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "c", "div_by_const_check.c"), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.strip().splitlines()
    assert len(lines) == 4
    for line in lines:
        assert "mismatches=0 " in line, line


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_newton_reciprocal_of_a_binary16_scale_is_correctly_rounded(tmp_path):
    exe = tmp_path / "recip_scale_newton"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "c", "recip_scale_newton.c"), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checked=158715 mismatches=0 " in r.stdout, r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_biased_code_decode_equals_the_two_step_decode(tmp_path):
    exe = tmp_path / "biased_decode_check"
    subprocess.run(["gcc", "-O3", "-march=native", "-fopenmp", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "c", "biased_decode_check.c"), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checked=2080309504 mismatches=0 unbiased_fma_mismatches=0 " in r.stdout, r.stdout


def test_raw_bit_order_of_ranges_that_hold_zero():
    """The kernels' group min/max for ranges that hold 0 (zero-aware and
    MSE: every lane's lo <= 0 <= hi) reduce the raw fp32 bit patterns: the
    largest unsigned pattern among values <= 0 is their minimum, and the
    largest signed pattern among values >= 0 (or -0) is their maximum; only
    the sign of a zero result may differ.  Checked on random groups mixing
    normal, subnormal and zero values of both signs, and on every pair of a
    set of edge values."""
    import numpy as np
    rng = np.random.default_rng(2026)
    edge = np.array([0.0, -0.0, 1e-45, 1e-38, 1.5e-38, 1.0, 3.4e38, 2.0 ** -149, 2.0 ** -126], np.float32)

    def reduce_lo(v):
        return np.max(v.view(np.uint32)).view(np.float32)

    def reduce_hi(v):
        return np.max(v.view(np.int32)).view(np.float32)

    def same(a, b):
        return a == b   # -0 == +0: only the sign of a zero may differ

    groups = []
    for _ in range(4000):
        m = rng.integers(1, 65)
        scale = 10.0 ** rng.uniform(-44, 38)
        v = (rng.standard_normal(m) * scale).astype(np.float32)
        v[rng.random(m) < 0.2] = 0.0
        v[rng.random(m) < 0.1] = -0.0
        groups.append(v)
    for a in edge:
        for b in edge:
            groups.append(np.array([a, b, -a, -b], np.float32))
    for v in groups:
        lo_vals = np.minimum(v, np.float32(0.0)).astype(np.float32)     # a lane's lo: min(0, ...)
        lo_vals[v == 0] = v[v == 0]                                      # keep the zeros' own signs
        hi_vals = np.maximum(v, np.float32(0.0)).astype(np.float32)
        assert np.all(lo_vals <= 0) and np.all(hi_vals >= 0)
        assert same(reduce_lo(lo_vals), lo_vals.min()), (v, reduce_lo(lo_vals), lo_vals.min())
        assert same(reduce_hi(hi_vals), hi_vals.max()), (v, reduce_hi(hi_vals), hi_vals.max())
    # a negative zero among zeros: the unsigned reduction returns a zero
    assert reduce_lo(np.array([0.0, -0.0], np.float32)) == 0.0
    assert reduce_hi(np.array([-0.0, -0.0], np.float32)) == 0.0
