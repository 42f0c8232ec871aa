"""Pins of the oracle's GEMMs and of its linear-layer composition.

Against: exact integer dot products (every E4M3 value is k*2^-9 and every E5M2
value k*2^-16 with integer k, so sums of products are exact in Python/int64
integers), Higham's bound for recursive fp32 summation, an identity-weight
special case, power-of-two block scales that keep every step exact, and the
float64 product X W^T (the method approximates the unquantized linear).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
QEXP = {"e4m3": 9, "e5m2": 16}


def int_table(fmt):
    """Integer k with value = k * 2^-QEXP, from torch's decode table."""
    v = torch.arange(256, dtype=torch.uint8).view(TORCH_DT[fmt]).double().numpy()
    k = np.where(np.isfinite(v), v * 2.0 ** QEXP[fmt], 0.0)
    assert np.all(k == np.round(k))
    return k.astype(np.int64)


def exact_gemm(A, fa, B, fb):
    """Exact sum_k A[i][k] B[j][k] as float64 mantissa-integers (object ints
    when they might not fit) times 2^-(QEXP[fa]+QEXP[fb])."""
    ka = int_table(fa)[A].astype(object)
    kb = int_table(fb)[B].astype(object)
    return ka.dot(kb.T), QEXP[fa] + QEXP[fb]


def codes_with_values(fmt, values, shape, rng):
    tab = torch.arange(256, dtype=torch.uint8).view(TORCH_DT[fmt]).float().numpy()
    codes = [int(np.where(tab == v)[0][0]) for v in values]
    return np.array(codes, np.uint8)[rng.integers(0, len(codes), size=shape)]


def finite_random_codes(fmt, shape, rng):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    bad = (c & 0x7F) == 0x7F if fmt == "e4m3" else (c & 0x7C) == 0x7C
    c[bad] = 0x38 if fmt == "e4m3" else 0x3C
    return c


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
def test_gemm_exact_when_sums_are_exact(fa, fb):
    rng = np.random.default_rng(0)
    vals = [-8.0, -3.0, -1.0, 0.0, 1.0, 2.0, 5.0, 7.0]
    A = codes_with_values(fa, vals, (96, 512), rng)
    B = codes_with_values(fb, vals, (80, 512), rng)
    C, C32 = oracle.gemm_tensor(A, fa, B, fb, 1.0, 1.0, want_f32=True)
    num, e = exact_gemm(A, fa, B, fb)
    ref = np.array(num, dtype=np.float64) * 2.0 ** -e
    assert np.array_equal(C32.astype(np.float64), ref)
    tref = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(C, tref)


@pytest.mark.parametrize("fa,fb,K", [("e4m3", "e4m3", 1024), ("e5m2", "e4m3", 768)])
def test_gemm_within_higham_bound(fa, fb, K):
    rng = np.random.default_rng(1)
    A = finite_random_codes(fa, (64, K), rng)
    B = finite_random_codes(fb, (48, K), rng)
    _, C32 = oracle.gemm_tensor(A, fa, B, fb, 1.0, 1.0, want_f32=True)
    num, e = exact_gemm(A, fa, B, fb)
    exact = np.array([[float(v) for v in row] for row in num]) * 2.0 ** -e
    absnum, _ = exact_gemm(A & 0x7F, fa, B & 0x7F, fb)
    sabs = np.array([[float(v) for v in row] for row in absnum]) * 2.0 ** -e
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    err = np.abs(C32.astype(np.float64) - exact)
    assert np.all(err <= gamma * sabs + 1e-300)


def test_gemm_scale_epilogue():
    rng = np.random.default_rng(2)
    vals = [-4.0, -1.0, 0.0, 1.0, 3.0, 6.0]
    A = codes_with_values("e4m3", vals, (64, 256), rng)
    B = codes_with_values("e4m3", vals, (32, 256), rng)
    sa, sb = np.float32(3.7e-3), np.float32(0.011)
    C, C32 = oracle.gemm_tensor(A, "e4m3", B, "e4m3", sa, sb, want_f32=True)
    num, e = exact_gemm(A, "e4m3", B, "e4m3")
    acc = (np.array(num, dtype=np.float64) * 2.0 ** -e).astype(np.float32)  # exact
    t = np.float32(sa * sb)
    assert np.array_equal(C32, acc * t)


def test_identity_weight():
    """W = c*I (c a power of two): Wq is the FMAX code on the diagonal, every
    output has a single product, and Y = bf16(fl32(448 dec(Xq) * t))."""
    K = 256
    x = synth.bits(synth.normal_bf16((128, K), 1.0, torch.Generator().manual_seed(4)))
    w = oracle.bf16_rne(np.eye(K, dtype=np.float32) * np.float32(0.125))
    y, ctx = oracle.linear_fwd(x, w, "tensor")
    wq = ctx["wq"]
    assert np.array_equal(wq["q_row"], np.eye(K, dtype=np.uint8) * 0x7E)
    xq = ctx["xq"]
    t = np.float32(xq["scale_inv"] * wq["scale_inv"])
    ref = oracle.bf16_rne((np.float32(448.0) * oracle.dec(xq["q_row"], "e4m3")) * t)
    assert np.array_equal(y, ref)
    # and it approximates 0.125 * X
    xf = oracle.dec_bf16(x).astype(np.float64)
    yf = oracle.dec_bf16(y).astype(np.float64)
    assert np.linalg.norm(yf - 0.125 * xf) / np.linalg.norm(0.125 * xf) < 0.05


@pytest.mark.parametrize("layout", ["fprop", "dgrad", "wgrad"])
def test_block_gemm_exact_with_power_of_two_scales(layout):
    rng = np.random.default_rng(5)
    I, J, K = 256, 256, 512
    KB = K // 128
    vals = [-3.0, -1.0, 0.0, 1.0, 2.0, 4.0]
    A = codes_with_values("e5m2", vals, (I, K), rng)
    B = codes_with_values("e4m3", vals, (J, K), rng)
    sA_full = (2.0 ** rng.integers(-2, 3, size=(I, KB))).astype(np.float32)
    sA = oracle.BlockScale(sA_full, 1, KB, 1)
    if layout == "fprop":      # B rows in 128-groups, scales [J/128, KB]
        arr = (2.0 ** rng.integers(-2, 3, size=(J // 128, KB))).astype(np.float32)
        sB = oracle.BlockScale(arr, 128, KB, 1)
        sB_full = np.repeat(arr, 128, axis=0)
    elif layout == "dgrad":    # transposed indexing: s[kb][r // 128]
        arr = (2.0 ** rng.integers(-2, 3, size=(KB, J // 128))).astype(np.float32)
        sB = oracle.BlockScale(arr, 128, 1, J // 128)
        sB_full = np.repeat(arr.T, 128, axis=0)
    else:                      # per row, 1x128
        arr = (2.0 ** rng.integers(-2, 3, size=(J, KB))).astype(np.float32)
        sB = oracle.BlockScale(arr, 1, KB, 1)
        sB_full = arr
    C, C32 = oracle.gemm_block(A, "e5m2", sA, B, "e4m3", sB, want_f32=True)
    ka = int_table("e5m2")[A]
    kb = int_table("e4m3")[B]
    ref = np.zeros((I, J))
    for b in range(KB):
        p = ka[:, b * 128:(b + 1) * 128] @ kb[:, b * 128:(b + 1) * 128].T  # exact int64
        ref += p * 2.0 ** -25 * sA_full[:, b][:, None] * sB_full[:, b][None, :]
    assert np.array_equal(C32.astype(np.float64), ref)


def test_block_gemm_equal_scales_close_to_tensor():
    rng = np.random.default_rng(6)
    A = finite_random_codes("e4m3", (128, 512), rng)
    B = finite_random_codes("e4m3", (128, 512), rng)
    s = np.float32(0.37)
    one = oracle.BlockScale(np.full((128, 4), s, np.float32), 1, 4, 1)
    _, cb = oracle.gemm_block(A, "e4m3", one, B, "e4m3", one, want_f32=True)
    _, ct = oracle.gemm_tensor(A, "e4m3", B, "e4m3", s, s, want_f32=True)
    assert np.allclose(cb, ct, rtol=1e-4, atol=1e-3 * np.abs(ct).max())


def test_sampled_equals_full():
    rng = np.random.default_rng(8)
    A = finite_random_codes("e5m2", (256, 384), rng)
    B = finite_random_codes("e4m3", (128, 384), rng)
    C = oracle.gemm_tensor(A, "e5m2", B, "e4m3", 0.5, 0.25)
    ii = rng.integers(0, 256, 500)
    jj = rng.integers(0, 128, 500)
    assert np.array_equal(oracle.gemm_tensor_sampled(A, "e5m2", B, "e4m3", 0.5, 0.25, ii, jj), C[ii, jj])
    sA = oracle.BlockScale(rng.uniform(0.1, 2, (256, 3)).astype(np.float32), 1, 3, 1)
    sB = oracle.BlockScale(rng.uniform(0.1, 2, (1, 3)).astype(np.float32), 128, 3, 1)
    Cb = oracle.gemm_block(A, "e5m2", sA, B, "e4m3", sB)
    assert np.array_equal(oracle.gemm_block_sampled(A, "e5m2", sA, B, "e4m3", sB, ii, jj), Cb[ii, jj])


@pytest.mark.parametrize("scaling", ["tensor", "block"])
def test_linear_approximates_float64(scaling):
    N, K, M = 512, 256, 384
    x, w, dy = synth.operands(N, K, M, seed=0, sigma_w=0.02, sigma_dy=1e-3)
    xb, wb, dyb = synth.bits(x), synth.bits(w), synth.bits(dy)
    y, ctx = oracle.linear_fwd(xb, wb, scaling)
    dx, dw, _ = oracle.linear_bwd(dyb, ctx)
    X, W, DY = (oracle.dec_bf16(t).astype(np.float64) for t in (xb, wb, dyb))

    def rel(a, b):
        return np.linalg.norm(oracle.dec_bf16(a).astype(np.float64) - b) / np.linalg.norm(b)
    assert rel(y, X @ W.T) < 0.06      # E4M3 x E4M3
    assert rel(dx, DY @ W) < 0.12      # E5M2 x E4M3
    assert rel(dw, DY.T @ X) < 0.12
    # a transposed or mis-indexed operand would be far off
    assert rel(dw, (DY.T @ X)[::-1]) > 0.5


def test_linear_reuses_forward_rounded_weight():
    """Passing the quantized weight back in (the cache) gives bitwise the same
    forward and backward as re-quantizing it."""
    x, w, dy = synth.operands(256, 256, 256, seed=3)
    xb, wb, dyb = synth.bits(x), synth.bits(w), synth.bits(dy)
    for scaling in ("tensor", "block"):
        y1, c1 = oracle.linear_fwd(xb, wb, scaling)
        wq = oracle.quantize_weight(wb, scaling)
        y2, c2 = oracle.linear_fwd(xb, None, scaling, wq=wq)
        assert np.array_equal(y1, y2)
        d1 = oracle.linear_bwd(dyb, c1)
        d2 = oracle.linear_bwd(dyb, c2)
        assert np.array_equal(d1[0], d2[0]) and np.array_equal(d1[1], d2[1])
