"""The seeded input recipes stay finite and follow their stated distributions
(CPU only)."""
import math

import numpy as np
import torch

from error_feedback_quant_amd import inputs


def f32(bits16: torch.Tensor) -> np.ndarray:
    return bits16.view(torch.bfloat16).float().numpy()


def test_laplace_transform_finite_at_the_extreme_draws():
    u = torch.tensor([0.0, 2.0 ** -24, 0.5, 1.0 - 2.0 ** -24], dtype=torch.float32)
    x = inputs.laplace_from_uniform(u)
    assert torch.isfinite(x).all()
    assert x[0] < 0 and x[-1] > 0 and x[2] == 0
    assert abs(float(x.abs().max()) - 24 * math.log(2)) < 1e-3
    assert (inputs._HALF_BELOW < 0.5) and torch.tensor(inputs._HALF_BELOW, dtype=torch.float32) < 0.5


def test_laplace_moments():
    x = f32(inputs.laplace(0, 1 << 22))
    assert np.isfinite(x).all()
    assert abs(x.mean()) < 0.01 and abs(np.abs(x).mean() - 1.0) < 0.01     # E|x| = b = 1


def test_single_outliers_and_chain_shapes():
    x = f32(inputs.single(0))
    assert x.size == 64 * 1024 and np.isfinite(x).all()
    assert (np.abs(x) > 8).sum() >= 40                       # the x20 outliers (66 drawn)
    y = f32(inputs.chain(0, 0, tokens=8, hidden=512))
    assert y.size == 8 * 512 and np.isfinite(y).all()
    z = f32(inputs.chain8(0, 0, tokens=64, hidden=1024))
    frac_small = (np.abs(z) < 1e-3).mean()
    assert 0.29 < frac_small < 0.33                          # 30 % near-zero mass (+1.6 % from N(0,0.05))
