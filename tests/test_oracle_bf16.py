"""Pins of the oracle's BF16 comparator GEMM and linear (the pages' baseline:
the same linears in BF16, "Native FP8 MLP reconstruction", isolated-linear
table).

Against: exact integer dot products (small integers are exact bf16 values
and their sums stay exact in fp32), the identity special case, Higham's
bound for recursive fp32 summation around the float64 product of the same
bf16 operands, and the linear's three products (Y = X W^T, dX = dY W,
dW = dY^T X) on non-square shapes, where a transposed operand cannot pass.
"""
import numpy as np
import torch

import oracle
import synth


def bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_exact_integer_sums():
    rng = np.random.default_rng(0)
    A = rng.integers(-8, 9, (96, 4096))
    B = rng.integers(-8, 9, (80, 4096))
    C, C32 = oracle.gemm_bf16(bf16_bits(A), bf16_bits(B), want_f32=True)
    exact = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.array_equal(C32.astype(np.float64), exact.astype(np.float64))
    assert np.array_equal(C, bf16_bits(exact.astype(np.float32)))


def test_identity_returns_the_operand():
    rng = np.random.default_rng(1)
    A = bf16_bits(rng.standard_normal((64, 256)) * 3)
    I = bf16_bits(np.eye(256))
    assert np.array_equal(oracle.gemm_bf16(A, I), A)


def _gamma_check(got_bits, A, B, K):
    """|fp32 sum - exact| <= gamma_K sum |a b|, then one bf16 rounding."""
    exact = A @ B.T
    n = K + 2
    g = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    bound = g * (np.abs(A) @ np.abs(B).T)
    a = np.abs(exact) + bound
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)
    err = np.abs(bf16_f64(got_bits) - exact)
    assert (err <= bound + 0.5 * ulp).all(), float((err / (bound + 0.5 * ulp)).max())


def test_random_within_higham_bound():
    rng = np.random.default_rng(2)
    A = bf16_bits(rng.standard_normal((128, 2048)))
    B = bf16_bits(rng.standard_normal((96, 2048)) * 0.02)
    C = oracle.gemm_bf16(A, B)
    _gamma_check(C, bf16_f64(A), bf16_f64(B), 2048)
    ii = rng.integers(0, 128, 300)
    jj = rng.integers(0, 96, 300)
    assert np.array_equal(oracle.gemm_bf16_sampled(A, B, ii, jj), C[ii, jj])


def test_linear_products_and_orientation():
    N, K, M = 384, 256, 640
    x, w, dy = (synth.bits(t) for t in synth.operands(N, K, M, seed=4, sigma_dy=1.0))
    y = oracle.linear_bf16_fwd(x, w)
    dx, dw = oracle.linear_bf16_bwd(dy, x, w)
    X, W, DY = bf16_f64(x), bf16_f64(w), bf16_f64(dy)
    assert y.shape == (N, M) and dx.shape == (N, K) and dw.shape == (M, K)
    _gamma_check(y, X, W, K)                     # Y = X W^T
    _gamma_check(dx, DY, W.T, M)                 # dX = dY W
    _gamma_check(dw, DY.T, X.T, N)               # dW = dY^T X
