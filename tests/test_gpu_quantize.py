"""Quantizer parity on the GPU: HIP kernels vs the CPU oracle, bit-exact on
every FP8 code and every fp32 scale.  Calls go through the C ABI."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from _util import to_np_u8

pytestmark = pytest.mark.gpu

FMT = {"e4m3": 0, "e5m2": 1}
SC = {"tensor": 0, "1x128": 1, "128x128": 2}


@pytest.fixture(scope="module")
def fp8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_mixed_precision_amax_amd as m
    m.lib()
    return m


def gpu_quant(fp8, x_bits, fmt, scaling, layouts=3):
    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    out = fp8.quantize(x, FMT[fmt], SC[scaling], layouts)
    torch.cuda.synchronize()
    return out


def compare(out, ref, scaling, layouts=3):
    f = lambda t: None if t is None else t.detach().cpu().numpy()
    if layouts & 1:
        assert np.array_equal(to_np_u8(out.q_row), ref["q_row"]), "row codes differ"
    if layouts & 2:
        assert np.array_equal(to_np_u8(out.q_col), ref["q_col"]), "col codes differ"
    if scaling == "tensor":
        assert f(out.scale)[0].view(np.uint32) == np.float32(ref["scale"]).view(np.uint32)
        assert f(out.scale_inv)[0].view(np.uint32) == np.float32(ref["scale_inv"]).view(np.uint32)
        a, b = f(out.amax)[0], np.float32(ref["amax"])
        assert (np.isnan(a) and np.isnan(b)) or a == b
    elif scaling == "1x128":
        if layouts & 1:
            assert np.array_equal(f(out.scale).view(np.uint32), ref["scale_row"].view(np.uint32))
            assert np.array_equal(f(out.scale_inv).view(np.uint32), ref["scale_inv_row"].view(np.uint32))
        if layouts & 2:
            assert np.array_equal(f(out.scale_col).view(np.uint32), ref["scale_col"].view(np.uint32))
            assert np.array_equal(f(out.scale_inv_col).view(np.uint32), ref["scale_inv_col"].view(np.uint32))
    else:
        assert np.array_equal(f(out.scale).view(np.uint32), ref["scale"].view(np.uint32))
        assert np.array_equal(f(out.scale_inv).view(np.uint32), ref["scale_inv"].view(np.uint32))


def normal_bits(shape, seed, sigma=1.0, outliers=0.0):
    g = torch.Generator().manual_seed(seed)
    return synth.bits(synth.normal_bf16(shape, sigma, g, outliers))


SHAPES = [(128, 128), (384, 640), (1024, 512), (640, 384)]   # 1, 15, 32, 15 tiles


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("scaling", ["tensor", "1x128", "128x128"])
@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_parity(fp8, fmt, scaling, shape):
    x = normal_bits(shape, zlib.crc32(repr((fmt, scaling, shape)).encode()) % 1000, outliers=0.01)
    out = gpu_quant(fp8, x, fmt, scaling)
    compare(out, oracle.quantize(x, fmt, scaling), scaling)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_every_bf16_pattern_encodes_like_oracle(fp8, fmt):
    """All 65536 bf16 patterns in one tensor: the NaNs make amax NaN, so the
    scale is 1 and every element is the plain encoding of its value
    (saturation, signed zero, subnormals, Inf and NaN included)."""
    x = np.arange(65536, dtype=np.uint16).reshape(512, 128)
    out = gpu_quant(fp8, x, fmt, "tensor")
    ref = oracle.quant_tensor(x, fmt)
    assert ref["scale"] == 1.0
    compare(out, ref, "tensor")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_every_finite_pattern_with_unit_scale(fp8, fmt):
    """Finite patterns only, with amax = FMAX so scale = 1 exactly: the NaN
    patch path is off and the hardware converter alone decides every code."""
    fmax_bits = {"e4m3": 0x43E0, "e5m2": 0x4760}[fmt]
    allb = np.arange(65536, dtype=np.uint16)
    keep = (allb & 0x7FFF) <= fmax_bits
    x = allb[keep]
    x = np.concatenate([x, np.full((-x.size) % (128 * 128), fmax_bits, np.uint16)]).reshape(-1, 128)
    out = gpu_quant(fp8, x, fmt, "tensor")
    ref = oracle.quant_tensor(x, fmt)
    assert ref["scale"] == 1.0
    compare(out, ref, "tensor")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_block_scales_over_many_magnitudes(fp8, fmt):
    """1x128 blocks whose amax spans the bf16 range: exercises the fp32
    division, the fp32 product and subnormal / saturating encodes."""
    rng = np.random.default_rng(5)
    x = normal_bits((512, 512), 77)
    xf = (x.astype(np.uint32) << 16).view(np.float32).reshape(512, 512)
    mult = (2.0 ** rng.uniform(-120, 120, size=(512, 4))).astype(np.float32)
    xf = (xf.reshape(512, 4, 128) * mult[:, :, None]).reshape(512, 512).astype(np.float32)
    bits = oracle.bf16_rne(xf)
    for scaling in ("1x128", "128x128", "tensor"):
        out = gpu_quant(fp8, bits, fmt, scaling)
        compare(out, oracle.quantize(bits, fmt, scaling), scaling)


@pytest.mark.parametrize("scaling", ["tensor", "1x128", "128x128"])
def test_zero_and_special_tensors(fp8, scaling):
    z = np.zeros((256, 256), np.uint16)
    z[5, 7] = 0x8000
    out = gpu_quant(fp8, z, "e4m3", scaling)
    compare(out, oracle.quantize(z, "e4m3", scaling), scaling)
    t = normal_bits((256, 256), 3)
    t[0, 0] = 0x7F80   # +Inf
    t[200, 131] = 0xFF80   # -Inf
    t[17, 250] = 0x7FC1   # NaN
    out = gpu_quant(fp8, t, "e5m2", scaling)
    compare(out, oracle.quantize(t, "e5m2", scaling), scaling)


@pytest.mark.parametrize("scaling", ["tensor", "1x128", "128x128"])
def test_fused_equals_separate_layouts(fp8, scaling):
    """One fused call writing both layouts gives the same bytes as a row-only
    and a col-only call ("fused output matches plain FP8 exactly")."""
    x = normal_bits((768, 384), 11, outliers=0.01)
    both = gpu_quant(fp8, x, "e4m3", scaling, 3)
    row = gpu_quant(fp8, x, "e4m3", scaling, 1)
    col = gpu_quant(fp8, x, "e4m3", scaling, 2)
    assert torch.equal(both.q_row, row.q_row)
    assert torch.equal(both.q_col, col.q_col)
    if scaling == "1x128":
        assert torch.equal(both.scale, row.scale) and torch.equal(both.scale_col, col.scale_col)
    else:
        assert torch.equal(both.scale, row.scale) and torch.equal(both.scale, col.scale)


def test_quantize_full_size_activation(fp8):
    """X of the 512 -> 2048 linear at N = 131072 tokens: all 64 Mi codes of
    both layouts and the scale, bit for bit."""
    N, K = 131072, 512
    g = torch.Generator().manual_seed(0)
    x = synth.bits(synth.normal_bf16((N, K), 1.0, g))
    out = gpu_quant(fp8, x, "e4m3", "tensor")
    compare(out, oracle.quant_tensor(x, "e4m3"), "tensor")
    out = gpu_quant(fp8, x, "e4m3", "1x128")
    compare(out, oracle.quant_block_1x128(x, "e4m3"), "1x128")
