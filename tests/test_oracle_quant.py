"""Pins of the oracle's amax, scale and quantizers.

Against: numpy's max(|x|) and float32 division (library routines), a
brute-force table encoder applied to numpy's float32 products, closed-form
invariants (power-of-two input scaling, the amax element hitting the FMAX
code, the half-ulp reconstruction bound) and the layout identities
(transposed layout = transpose; 1x128 column blocks = row blocks of X^T).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle_codec import brute_force_encode

FMAX = {"e4m3": 448.0, "e5m2": 57344.0}
FMAX_CODE = {"e4m3": 0x7E, "e5m2": 0x7B}


def bf16_bits(shape, seed, sigma=1.0, outliers=0.0):
    g = torch.Generator().manual_seed(seed)
    return synth.bits(synth.normal_bf16(shape, sigma, g, outliers))


def f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_amax_matches_numpy_and_is_order_free():
    x = bf16_bits((256, 384), 1, outliers=0.01)
    ref = np.abs(f32(x)).max()
    assert oracle.amax_bf16(x) == ref
    perm = np.random.default_rng(0).permutation(x.size)
    assert oracle.amax_bf16(x.reshape(-1)[perm]) == ref
    y = x.copy()
    y[7, 11] = 0x7FC1  # a NaN
    assert np.isnan(oracle.amax_bf16(y))
    assert oracle.amax_bf16(np.array([0x8000, 0x0000], np.uint16)) == 0.0  # -0, +0


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_scale_matches_numpy_division(fmt):
    rng = np.random.default_rng(3)
    am = np.concatenate([np.exp(rng.uniform(-80, 80, 20000)).astype(np.float32),
                         (np.arange(1, 65536, dtype=np.uint32) << 16).view(np.float32)])
    am = am[np.isfinite(am) & (am > 0)]
    for a in am[:: max(1, am.size // 4000)]:
        s, si = oracle.scale_from_amax(a, fmt)
        with np.errstate(over="ignore"):
            ref = np.float32(FMAX[fmt]) / np.float32(a)
        if np.isinf(ref):
            ref = np.finfo(np.float32).max
        assert s == ref and si == np.float32(1.0) / ref


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_scale_special_cases(fmt):
    for a in (0.0, np.inf, np.nan):
        s, si = oracle.scale_from_amax(a, fmt)
        assert s == 1.0 and si == 1.0
    s, si = oracle.scale_from_amax(np.float32(1e-39), fmt)  # subnormal amax: overflow
    assert s == np.finfo(np.float32).max
    assert si == np.float32(1.0) / np.finfo(np.float32).max


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quant_tensor_against_library_pieces(fmt):
    x = bf16_bits((384, 256), 5)
    r = oracle.quant_tensor(x, fmt)
    amax = np.abs(f32(x)).max()
    s = np.float32(FMAX[fmt]) / np.float32(amax)
    assert r["amax"] == amax and r["scale"] == s and r["scale_inv"] == np.float32(1) / s
    ref = brute_force_encode(f32(x) * s, fmt)
    assert np.array_equal(r["q_row"], ref)
    assert np.array_equal(r["q_col"], ref.T)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quant_tensor_amax_element_hits_fmax_and_half_ulp(fmt):
    x = bf16_bits((256, 512), 9, outliers=0.01)
    r = oracle.quant_tensor(x, fmt, col=False)
    xv = f32(x).astype(np.float64)
    i = np.argmax(np.abs(xv))
    assert (r["q_row"].reshape(-1)[i] & 0x7F) == FMAX_CODE[fmt]
    d = oracle.dec(r["q_row"], fmt).astype(np.float64)
    v = xv * np.float64(r["scale"])
    # half an FP8 spacing at |v| (spacing 2^(e-m), e clamped at the min normal)
    mb = 3 if fmt == "e4m3" else 2
    emin = -6 if fmt == "e4m3" else -14
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(v), 1e-300))), emin)
    half = 2.0 ** (e - mb) / 2
    # the fp32 product adds at most one fp32 rounding of v
    assert np.all(np.abs(d - v) <= half * (1 + 1e-6) + np.abs(v) * 2.0 ** -24)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("k", [-3, 1, 4])
def test_power_of_two_invariance(fmt, k):
    """Scaling X by 2^k (no overflow/underflow) leaves every code unchanged and
    multiplies scale_inv by exactly 2^k."""
    x = bf16_bits((128, 256), 11)
    xk = oracle.bf16_rne(f32(x) * np.float32(2.0 ** k))
    assert np.array_equal(f32(xk), f32(x) * np.float32(2.0 ** k))
    a = oracle.quant_tensor(x, fmt)
    b = oracle.quant_tensor(xk, fmt)
    assert np.array_equal(a["q_row"], b["q_row"])
    assert b["scale_inv"] == a["scale_inv"] * np.float32(2.0 ** k)
    a = oracle.quant_block_1x128(x, fmt)
    b = oracle.quant_block_1x128(xk, fmt)
    assert np.array_equal(a["q_row"], b["q_row"]) and np.array_equal(a["q_col"], b["q_col"])
    assert np.array_equal(b["scale_inv_row"], a["scale_inv_row"] * np.float32(2.0 ** k))


def test_quant_zero_tensor():
    x = np.zeros((128, 128), np.uint16)
    x[3, 5] = 0x8000  # -0.0
    r = oracle.quant_tensor(x, "e4m3")
    assert r["scale"] == 1.0 and r["scale_inv"] == 1.0
    assert r["q_row"][3, 5] == 0x80 and (r["q_row"].sum() == 0x80)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_block_1x128_rows_against_library_pieces(fmt):
    x = bf16_bits((256, 384), 21, outliers=0.01)
    r = oracle.quant_block_1x128(x, fmt)
    xf = f32(x)
    blocks = xf.reshape(256, 3, 128)
    amax = np.abs(blocks).max(axis=2)
    s = np.float32(FMAX[fmt]) / amax.astype(np.float32)
    assert np.array_equal(r["scale_row"], s)
    assert np.array_equal(r["scale_inv_row"], np.float32(1) / s)
    ref = brute_force_encode((blocks * s[:, :, None]).reshape(256, 384), fmt)
    assert np.array_equal(r["q_row"], ref)
    # every block's largest element encodes to +-FMAX
    q = r["q_row"].reshape(256, 3, 128)
    arg = np.abs(blocks).argmax(axis=2)
    picked = np.take_along_axis(q, arg[:, :, None], axis=2)[..., 0]
    assert np.all((picked & 0x7F) == FMAX_CODE[fmt])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_block_1x128_cols_are_rows_of_transpose(fmt):
    x = bf16_bits((384, 256), 22, outliers=0.01)
    r = oracle.quant_block_1x128(x, fmt)
    t = oracle.quant_block_1x128(np.ascontiguousarray(x.T), fmt, col=False)
    assert np.array_equal(r["q_col"], t["q_row"])
    assert np.array_equal(r["scale_col"], t["scale_row"])
    assert np.array_equal(r["scale_inv_col"], t["scale_inv_row"])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_block_128x128(fmt):
    x = bf16_bits((384, 256), 23, outliers=0.01)
    r = oracle.quant_block_128x128(x, fmt)
    assert np.array_equal(r["q_col"], r["q_row"].T)
    xf = f32(x)
    for rb in range(3):
        for cb in range(2):
            tile = x[rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128]
            t = oracle.quant_tensor(tile, fmt, col=False)  # one tile == tensorwise on it
            assert r["scale"][rb, cb] == t["scale"] and r["scale_inv"][rb, cb] == t["scale_inv"]
            assert np.array_equal(r["q_row"][rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128], t["q_row"])
            amax = np.abs(xf[rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128]).max()
            assert t["scale"] == np.float32(FMAX[fmt]) / amax


def test_fused_equals_separate_layouts():
    x = bf16_bits((256, 384), 31)
    for fn in (oracle.quant_tensor, oracle.quant_block_1x128, oracle.quant_block_128x128):
        both = fn(x, "e4m3")
        row = fn(x, "e4m3", col=False)
        col = fn(x, "e4m3", row=False)
        assert np.array_equal(both["q_row"], row["q_row"])
        assert np.array_equal(both["q_col"], col["q_col"])
