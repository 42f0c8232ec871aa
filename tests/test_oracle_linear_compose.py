"""Pins of the oracle's linear-layer composition: which codes and which
scale factors each of its three GEMMs consumes.

The oracle's Y, dX and dW are compared with float64 products of operands
dequantized here, independently of the oracle's GEMM scale descriptors: every
FP8 code is decoded by torch's OCP table and multiplied by the factor of the
block it lies in, written out with plain numpy broadcasting (1x128 blocks of
the row layout along the columns, of the col layout along the rows; 128x128
weight tiles read in place for the row layout and transposed for the col
layout).  The only difference left is the oracle's fp32 rounding, bounded by
Higham's gamma bound (recursive summation, plus the products of scale
factors and the final bf16 rounding).

The weight carries one 128x128 tile scaled by 100 at an off-diagonal position
and the activations / gradients 1% outliers scaled by 100, so that reading a
factor of the wrong block (a transposed tile index, the row-layout scales in
place of the col-layout ones, a block stride off by one) changes the affected
outputs by far more than the bound.  The recipe is "Native FP8 MLP
reconstruction" (implementation paragraph: X and W codes of the forward pass
reused in the backward pass, the gradient quantized on its own) with the
block scaling of TransformerEngine issue 2852 (opening post).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def decode(codes, fmt):
    """FP8 codes -> float64 through torch's table (not the oracle's)."""
    tab = torch.arange(256, dtype=torch.uint8).view(TORCH_DT[fmt]).double().numpy()
    return tab[codes]


def rows_1x128(q, fmt, sinv):
    """Dequantized [R, C] whose factors are per (row, 128-column block):
    sinv [R, C/128]."""
    return decode(q, fmt) * np.repeat(np.asarray(sinv, np.float64), 128, axis=1)


def tiles_128x128(q, fmt, sinv, transposed):
    """Dequantized weight layout with factors per 128x128 tile of the
    source: sinv [R/128, C/128] of the source W [R, C]; the col layout
    [C, R] reads the tile (r // 128, c // 128) at position (c, r)."""
    t = np.asarray(sinv, np.float64)
    if transposed:
        t = t.T
    return decode(q, fmt) * np.kron(t, np.ones((128, 128)))


def tensorwise(q, fmt, sinv):
    return decode(q, fmt) * np.float64(sinv)


def gamma_bound(Ad, Bd, K):
    """Bound on |oracle fp32 result - exact| for C = Ad Bd^T: recursive
    summation of K products with per-block promotion and one rounding of each
    scale product, all well inside gamma_(K + 8) times sum |a b|."""
    n = K + 8
    u = 2.0 ** -24
    return (n * u / (1 - n * u)) * (np.abs(Ad) @ np.abs(Bd).T)


def check_close(got_bits, exact, bound, name):
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = np.abs(exact) + bound
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)
    lim = bound + 0.5 * ulp            # fp32 error, then one bf16 rounding
    err = np.abs(got - exact)
    worst = float((err / lim).max())
    assert (err <= lim).all(), (name, worst, np.argwhere(err > lim)[:5])
    return worst


def block_operands(N, K, M, seed):
    g = torch.Generator().manual_seed(seed)
    x = synth.normal_bf16((N, K), 1.0, g, outlier_frac=0.01)
    w = torch.randn((M, K), generator=g)
    w[0:128, 256:384] *= 100.0            # tile (0, 2): off the diagonal
    w = w.to(torch.bfloat16)
    dy = synth.normal_bf16((N, M), 1.0, g, outlier_frac=0.01)
    return synth.bits(x), synth.bits(w), synth.bits(dy)


@pytest.mark.parametrize("N,K,M", [(512, 512, 512), (256, 384, 640)])
def test_block_linear_against_independent_dequantization(N, K, M):
    x, w, dy = block_operands(N, K, M, seed=11)
    y, ctx = oracle.linear_fwd(x, w, "block")
    dx, dw, dyq = oracle.linear_bwd(dy, ctx)
    xq, wq = ctx["xq"], ctx["wq"]
    # the outlier tile really has its own factor
    assert wq["scale_inv"][0, 2] > 20 * np.median(wq["scale_inv"])

    Xd = rows_1x128(xq["q_row"], "e4m3", xq["scale_inv_row"])          # [N, K]
    Wd = tiles_128x128(wq["q_row"], "e4m3", wq["scale_inv"], False)     # [M, K]
    WdT = tiles_128x128(wq["q_col"], "e4m3", wq["scale_inv"], True)     # [K, M]
    dYd = rows_1x128(dyq["q_row"], "e5m2", dyq["scale_inv_row"])        # [N, M]
    dYdT = rows_1x128(dyq["q_col"], "e5m2", dyq["scale_inv_col"])       # [M, N]
    XdT = rows_1x128(xq["q_col"], "e4m3", xq["scale_inv_col"])          # [K, N]
    # the two layouts of one tensor dequantize to nearly the same values
    assert np.allclose(WdT, Wd.T, rtol=0, atol=0)                        # 128x128: same codes, same tile
    assert np.abs(XdT - Xd.T).max() <= 2.0 ** -3 * np.abs(Xd).max()

    for name, got, A, B, Kc in [("Y", y, Xd, Wd, K), ("dX", dx, dYd, WdT, M), ("dW", dw, dYdT, XdT, N)]:
        exact = A @ B.T
        check_close(got, exact, gamma_bound(A, B, Kc), "block " + name)


def test_tensor_linear_against_independent_dequantization():
    N, K, M = 384, 512, 640
    x, w, dy = (synth.bits(t) for t in synth.operands(N, K, M, seed=3))
    y, ctx = oracle.linear_fwd(x, w, "tensor")
    dx, dw, dyq = oracle.linear_bwd(dy, ctx)
    xq, wq = ctx["xq"], ctx["wq"]
    Xd = tensorwise(xq["q_row"], "e4m3", xq["scale_inv"])
    Wd = tensorwise(wq["q_row"], "e4m3", wq["scale_inv"])
    WdT = tensorwise(wq["q_col"], "e4m3", wq["scale_inv"])
    dYd = tensorwise(dyq["q_row"], "e5m2", dyq["scale_inv"])
    dYdT = tensorwise(dyq["q_col"], "e5m2", dyq["scale_inv"])
    XdT = tensorwise(xq["q_col"], "e4m3", xq["scale_inv"])
    for name, got, A, B, Kc in [("Y", y, Xd, Wd, K), ("dX", dx, dYd, WdT, M), ("dW", dw, dYdT, XdT, N)]:
        check_close(got, A @ B.T, gamma_bound(A, B, Kc), "tensor " + name)
