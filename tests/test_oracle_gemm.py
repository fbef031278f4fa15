"""Pins for the oracle's matmul step and its fused matmul + entry pass (CPU).

The partial sums x = bf16(A W^T) of a row-parallel layer are the message of
the all-reduce (Echo paper card Fig. 2(a)); the fused call is that matmul
followed by the push step (article "The cancellation rule": folding the
compensator into the entry pass leaves the results as they were).

Pins: exact integer dot products (pure Python) with W in [N, K] layout, so a
transposed operand or a swapped index fails; the bf16 rounding of a sum
(ties to even, both directions); and the fused call's outputs against its
two steps, own rows written, other rows left alone.
"""
import numpy as np
import pytest

import oracle
from error_feedback_quant_amd import inputs


def bits_of(vals):
    return oracle.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_matmul_is_the_integer_dot_product_per_row_and_weight_row():
    rng = np.random.default_rng(200)
    M, N, K = 5, 3, 64
    A = rng.integers(-7, 8, size=(M, K))
    W = rng.integers(-7, 8, size=(N, K))
    x = oracle.matmul_bf16(bits_of(A), bits_of(W))
    assert x.shape == (M * N,)
    want = [sum(int(A[m][k]) * int(W[j][k]) for k in range(K)) for m in range(M) for j in range(N)]
    assert np.array_equal(x, bits_of(want))
    # the transposed reading (sum_k A[m][k] W[k][j]) is a different matrix
    assert not np.array_equal(oracle.matmul_bf16(bits_of(A[:, :3]), bits_of(W[:, :3])),
                              bits_of((A[:, :3] @ W[:, :3].T).T.reshape(-1)[:M * N]))


def test_matmul_rounds_the_sum_to_bf16_ties_to_even():
    # bf16 keeps 8 significant bits: 257 and 259 are ties between neighbours
    A = bits_of([[1.0, 1.0]])
    for w, want in (([256.0, 1.0], 256.0), ([258.0, 1.0], 260.0), ([256.0, 3.0], 260.0)):
        x = oracle.matmul_bf16(A, bits_of([w]))
        assert np.array_equal(x, bits_of([want])), (w, x)


def test_matmul_of_fractional_operands():
    # products of bf16 values are exact in float64; a sum below 2^-126 stays
    # a (fp32) subnormal before the bf16 rounding
    A = bits_of([[2.0 ** -70, 2.0 ** -70]])
    W = bits_of([[2.0 ** -60, 2.0 ** -61]])
    x = oracle.matmul_bf16(A, W)
    assert np.array_equal(x, bits_of([2.0 ** -130 + 2.0 ** -131]))


@pytest.mark.parametrize("flags", [0, oracle.ERR_NEGATED, oracle.X_ALL | oracle.Q_NAIVE])
@pytest.mark.parametrize("P,rank", [(4, 1), (2, 0), (1, 0)])
def test_fused_call_is_matmul_then_push(P, rank, flags):
    M, N, K = 128 * P, 256, 64
    a, w = (inputs.as_numpy_u16(t) for t in inputs.tp_operands(rank, M, N, K, "int"))
    a, w = a.reshape(M, K), w.reshape(N, K)
    n = M * N
    rng = np.random.default_rng(210 + P)
    comp = (rng.standard_normal(n) * 0.1).astype(np.float32)
    codes = np.zeros(n // 2, np.uint8); params = np.zeros(2 * n // 128, np.uint16)
    err = np.full(n, 7.0, np.float32); x_out = np.full(n, 0xBEEF, np.uint16)
    x = oracle.gemm_quantize_ef(a, w, comp, P, rank, 4, codes, params, err, x_out, flags)
    assert np.array_equal(x, oracle.matmul_bf16(a, w))
    wc = np.zeros_like(codes); wp = np.zeros_like(params); we = np.full(n, 7.0, np.float32)
    oracle.quantize_ef(x, comp, n, P, rank, 0, n // P, 4, 128, wc, wp, we, flags & ~oracle.X_ALL)
    assert np.array_equal(codes, wc) and np.array_equal(params, wp) and np.array_equal(err, we)
    S = n // P
    own = slice(rank * S, (rank + 1) * S)
    assert np.array_equal(x_out[own], x[own])
    rest = np.ones(n, bool); rest[own] = False
    if flags & oracle.X_ALL:
        assert np.array_equal(x_out, x)
    else:
        assert np.all(x_out[rest] == 0xBEEF)
