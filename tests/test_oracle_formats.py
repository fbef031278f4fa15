"""Pins for the oracle's number-format conversions (CPU only).

binary16 is where the per-group scale and zero point live (PhantomByte article
on Echo, "The cancellation rule": each group's parameters travel at half
precision); bfloat16 is the message format.  The oracle's converters are written
from the IEEE 754 definitions; here they are checked against independent
library conversions (torch's and numpy's CPU casts, both round to nearest even).
"""
import numpy as np
import pytest
import torch

import oracle


def _torch_f16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(f32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def test_f16_exhaustive_over_every_rounding_binade():
    """Every positive binary32 whose binade rounds to something other than
    0 or infinity in binary16 (2^-27 <= v < 2^17): 45 * 2^23 values."""
    lo_field, hi_field = 127 - 27, 127 + 17
    step = 1 << 23
    for e in range(lo_field, hi_field):
        u = (np.arange(step, dtype=np.uint32) | np.uint32(e << 23))
        f = u.view(np.float32)
        got = oracle.f32_to_f16_bits(f)
        want = _torch_f16_bits(f)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (e, hex(int(u[bad[0]])), hex(int(got[bad[0]])), hex(int(want[bad[0]])))


def test_f16_sampled_everywhere_including_signs_and_specials():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001, 0x807FFFFF,
                         0x477FE000, 0x477FEFFF, 0x477FF000, 0x477FF001,   # around 65504 / 65520
                         0x33000000, 0x33000001, 0x32FFFFFF, 0x33800000,   # 2^-25 and 2^-24
                         0x387FC000, 0x387FE000, 0x38800000], dtype=np.uint32)
    u = np.concatenate([u, specials, specials | np.uint32(0x80000000)])
    f = u.view(np.float32)
    got = oracle.f32_to_f16_bits(f)
    want = _torch_f16_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_f16_to_f32_all_patterns():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = h.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_bits_to_f32(int(v)) for v in h], dtype=np.float32)
    finite = np.isfinite(want)
    assert np.array_equal(got[finite].view(np.uint32), want[finite].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got), np.isinf(want))


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(2)
    u = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    # explicit ties: low half exactly 0x8000 with even and odd upper halves
    ties = (rng.integers(0, 1 << 16, size=4096, dtype=np.uint32) << 16) | np.uint32(0x8000)
    u = np.concatenate([u, ties, ties - 1, ties + 1])
    f = u.view(np.float32)
    keep = np.isfinite(f)
    f = f[keep]
    got = oracle.f32_to_bf16_bits(f)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
