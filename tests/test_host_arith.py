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
