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


def test_tp_operands_recipes():
    a, w = inputs.tp_operands(0, 64, 32, 256, "int")
    A, W = f32(a.reshape(-1)), f32(w.reshape(-1))
    assert a.shape == (64, 256) and w.shape == (32, 256)
    assert np.array_equal(A, np.round(A)) and A.min() >= -4 and A.max() <= 4
    assert np.array_equal(W, np.round(W)) and W.min() >= -3 and W.max() <= 3
    # every product and partial sum of a row is an integer below 2^24: exact in fp32
    assert 256 * 4 * 3 < 2 ** 24
    a, w = inputs.tp_operands(1, 256, 128, 1024, "normal")
    A, W = f32(a.reshape(-1)), f32(w.reshape(-1))
    assert abs(A.std() - 1.0) < 0.02 and abs(W.std() * math.sqrt(1024) - 1.0) < 0.03
    # the partial sums of a random-init layer have unit scale
    x = (A.reshape(256, 1024).astype(np.float64) @ W.reshape(128, 1024).astype(np.float64).T)
    assert 0.9 < x.std() < 1.1
    a, w = inputs.tp_operands(2, 64, 32, 4096, "ternary")
    A, W = f32(a.reshape(-1)), f32(w.reshape(-1))
    assert set(np.unique(A)) == {-1.0, 0.0, 1.0} and set(np.unique(W)) == {-1.0, 0.0, 1.0}
    assert abs(np.mean(A == 0) - 1 / 3) < 0.01
    # |partial sum| <= K: exact in fp32 for every K below 2^24
    # seeded: the same rank gives the same draw, another rank a different one
    assert torch.equal(inputs.tp_operands(1, 8, 8, 64)[0], inputs.tp_operands(1, 8, 8, 64)[0])
    assert not torch.equal(inputs.tp_operands(1, 8, 8, 64)[0], inputs.tp_operands(2, 8, 8, 64)[0])
