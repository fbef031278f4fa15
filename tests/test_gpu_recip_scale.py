"""The kernels' reciprocal of a binary16 scale on the GPU, for every scale.

Every quantizer multiplies by 1/s, correctly rounded, where s is the group's
binary16 scale (2^-24 <= s <= 65504 after the clamps).  The kernels compute
it as one Newton step from the hardware reciprocal (echo::recip_scale).  A
test-only device library (tests/c/recip_scale_check.hip, built with the
library's flags) evaluates that function for all 65536 binary16 patterns;
each of the 31743 positive finite ones must give the IEEE quotient 1/s,
which numpy's float32 division is."""
import ctypes
import os

import numpy as np
import pytest
import torch

from _helpers import say

pytestmark = pytest.mark.gpu
LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "librecip_scale_check.so")


def test_recip_scale_is_the_ieee_quotient_for_every_binary16_scale():
    assert torch.cuda.is_available()
    assert os.path.exists(LIB), f"{LIB} is not built (build() compiles it)"
    lib = ctypes.CDLL(LIB)
    lib.recip_scale_all.argtypes = [ctypes.c_void_p]
    lib.recip_scale_all.restype = ctypes.c_int
    out = np.zeros(1 << 16, np.uint32)
    say("recip_scale", "all binary16 patterns")
    rc = lib.recip_scale_all(out.ctypes.data)
    assert rc == 0, f"HIP error {rc}"
    h = np.arange(1, 0x7C00, dtype=np.uint16)
    s = h.view(np.float16).astype(np.float32)
    want = (np.float32(1.0) / s).view(np.uint32)
    got = out[1:0x7C00]
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(h[i])), hex(int(got[i])), hex(int(want[i]))) for i in bad[:8]]
