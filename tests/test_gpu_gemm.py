"""FP8 GEMM parity on the GPU: the HIP matrix-core GEMM vs the oracle's
fp32-accumulated GEMM, within the BF16 tolerance of tests/_util.py, for every
operand-format pair the linear uses, tensorwise and block-scaled, on shapes
that span several tiles, half-full edge tiles and split-K."""
import numpy as np
import pytest
import torch

import oracle
from _util import check_gemm, to_np_u16

pytestmark = pytest.mark.gpu

FMT = {"e4m3": 0, "e5m2": 1}


@pytest.fixture(scope="module")
def fp8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_mixed_precision_amax_amd as m
    m.lib()
    return m


def rand_codes(fmt, shape, rng):
    """Codes of quantized normal data (finite), like the linear produces."""
    v = (rng.standard_normal(shape) * (100.0 if fmt == "e4m3" else 8000.0)).astype(np.float32)
    return oracle.enc(v, fmt)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


TENSOR_CASES = [
    # I, J, K, fa, fb
    (256, 256, 128, "e4m3", "e4m3"),
    (384, 640, 512, "e4m3", "e4m3"),     # half-full edge tiles in i and j
    (1024, 512, 512, "e5m2", "e4m3"),
    (512, 384, 1024, "e5m2", "e4m3"),
    (256, 256, 16384, "e5m2", "e4m3"),   # split-K
    (128, 128, 4096, "e4m3", "e5m2"),
    (640, 128, 2048, "e5m2", "e5m2"),
]


@pytest.mark.parametrize("I,J,K,fa,fb", TENSOR_CASES)
def test_gemm_tensorwise(fp8, I, J, K, fa, fb):
    rng = np.random.default_rng(I * 7 + J * 3 + K)
    A = rand_codes(fa, (I, K), rng)
    B = rand_codes(fb, (J, K), rng)
    sa, sb = np.float32(rng.uniform(1e-3, 1e-2)), np.float32(rng.uniform(1e-4, 1e-2))
    ref = oracle.gemm_tensor(A, fa, B, fb, sa, sb)
    ta, tb = dev(A), dev(B)
    tsa = torch.tensor([sa], device="cuda")
    tsb = torch.tensor([sb], device="cuda")
    c = fp8.gemm(ta, FMT[fa], fp8.gemm_scale(tsa), tb, FMT[fb], fp8.gemm_scale(tsb))
    torch.cuda.synchronize()
    print(check_gemm(to_np_u16(c), ref, A, fa, B, fb, np.float32(sa * sb), K, "gemm %dx%dx%d" % (I, J, K)), flush=True)


BLOCK_CASES = [
    # I, J, K, fa, fb, A layout, B layout:
    #   "row":  1x128 factors [rows, K/128] row-major
    #   "rowT": 1x128 factors stored block-major [K/128, rows] (what the quantizer writes)
    #   "blk":  128x128 factors [rows/128, K/128];  "blkT": transposed
    (256, 256, 512, "e4m3", "e4m3", "row", "blk"),
    (384, 640, 256, "e4m3", "e4m3", "row", "blk"),
    (512, 256, 512, "e5m2", "e4m3", "row", "blkT"),
    (384, 384, 384, "e5m2", "e4m3", "row", "row"),
    (256, 128, 16384, "e5m2", "e4m3", "row", "row"),     # split-K
    (640, 384, 1152, "e5m2", "e4m3", "rowT", "rowT"),    # ragged last tile, block-major factors
    (384, 512, 768, "e4m3", "e5m2", "blk", "rowT"),      # 128x128 factors on the A side
    (128, 256, 4096, "e4m3", "e4m3", "rowT", "blkT"),    # one half-full tile, split-K
]


def block_factors(layout, rows, KB, rng):
    """(array, oracle.BlockScale, per-row factors [rows, KB]) for one operand."""
    if layout == "row":
        arr = rng.uniform(1e-3, 1e-1, (rows, KB)).astype(np.float32)
        return arr, oracle.BlockScale(arr, 1, KB, 1), arr
    if layout == "rowT":
        arr = rng.uniform(1e-3, 1e-1, (KB, rows)).astype(np.float32)
        return arr, oracle.BlockScale(arr, 1, 1, rows), arr.T
    if layout == "blk":
        arr = rng.uniform(1e-3, 1e-1, (rows // 128, KB)).astype(np.float32)
        return arr, oracle.BlockScale(arr, 128, KB, 1), np.repeat(arr, 128, axis=0)
    arr = rng.uniform(1e-3, 1e-1, (KB, rows // 128)).astype(np.float32)
    return arr, oracle.BlockScale(arr, 128, 1, rows // 128), np.repeat(arr.T, 128, axis=0)


@pytest.mark.parametrize("I,J,K,fa,fb,al,bl", BLOCK_CASES)
def test_gemm_block(fp8, I, J, K, fa, fb, al, bl):
    rng = np.random.default_rng(I + J * 5 + K * 11)
    KB = K // 128
    A = rand_codes(fa, (I, K), rng)
    B = rand_codes(fb, (J, K), rng)
    sA_arr, sA, sA_full = block_factors(al, I, KB, rng)
    sB_arr, sB, sB_full = block_factors(bl, J, KB, rng)
    ref = oracle.gemm_block(A, fa, sA, B, fb, sB)
    tsa, tsb = dev(sA_arr), dev(sB_arr)
    c = fp8.gemm(dev(A), FMT[fa], fp8.gemm_scale(tsa, sA.group, sA.stride_r, sA.stride_kb),
                 dev(B), FMT[fb], fp8.gemm_scale(tsb, sB.group, sB.stride_r, sB.stride_kb))
    torch.cuda.synchronize()
    t = (np.ascontiguousarray(sA_full), np.ascontiguousarray(sB_full))
    print(check_gemm(to_np_u16(c), ref, A, fa, B, fb, t, K, "block gemm %dx%dx%d %s %s" % (I, J, K, al, bl)), flush=True)


def test_gemm_identity_places_every_element(fp8):
    """B = FMAX code on the diagonal: C[i][j] = bf16(fl32(448 * dec(A[i][j])) * t),
    one product per output, so indexing and layout errors cannot hide."""
    K = 512
    rng = np.random.default_rng(3)
    A = rand_codes("e4m3", (384, K), rng)
    B = (np.eye(K, dtype=np.uint8) * 0x7E)
    sa, sb = np.float32(0.37), np.float32(0.011)
    ref = oracle.gemm_tensor(A, "e4m3", B, "e4m3", sa, sb)
    c = fp8.gemm(dev(A), 0, fp8.gemm_scale(torch.tensor([sa], device="cuda")), dev(B), 0,
                 fp8.gemm_scale(torch.tensor([sb], device="cuda")))
    torch.cuda.synchronize()
    got = to_np_u16(c)
    # single product: the fp32 sum is exact; at most the epilogue order differs
    assert np.abs(got.astype(np.int32) - ref.astype(np.int32)).max() <= 1


def test_gemm_deterministic(fp8):
    rng = np.random.default_rng(9)
    A = dev(rand_codes("e5m2", (512, 8192), rng))
    B = dev(rand_codes("e4m3", (256, 8192), rng))
    s = fp8.gemm_scale(torch.tensor([1e-3], device="cuda"))
    c1 = fp8.gemm(A, 1, s, B, 0, s)
    c2 = fp8.gemm(A, 1, s, B, 0, s)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


def finite_codes(fmt, shape, rng):
    """Uniformly random finite codes over the whole format (every binade,
    subnormals and both signs): NaN (E4M3) or Inf/NaN (E5M2) patterns are
    moved to the largest finite code of their sign."""
    b = rng.integers(0, 256, int(np.prod(shape)), dtype=np.uint8)
    if fmt == "e4m3":
        b[(b & 0x7F) == 0x7F] -= 1
    else:
        b[(b & 0x7C) == 0x7C] &= 0xFB
    return b.reshape(shape)


KMAX = (1 << 23) - 128   # the longest contraction the library accepts


@pytest.mark.parametrize("scaling", ["tensor", "block", "block_wide"])
def test_gemm_longest_contraction(fp8, scaling):
    """K = 2^23 - 128 (one 128 x 128 output tile, the most split-K slices),
    operands drawn over every finite code: sampled outputs against the oracle
    and the matrix-core emulation.  Offsets inside a tile reach ~2^31 bytes
    here, the edge of the 32-bit buffer offsets the kernels use."""
    I = J = 128
    print("longest contraction", scaling, I, J, KMAX, flush=True)
    rng = np.random.default_rng(23)
    A = finite_codes("e5m2", (I, KMAX), rng)
    B = finite_codes("e4m3", (J, KMAX), rng)
    ii = rng.integers(0, I, 16)
    jj = rng.integers(0, J, 16)
    if scaling == "tensor":
        sa, sb = np.float32(2.0 ** -17), np.float32(3.0e-6)
        c = fp8.gemm(dev(A), 1, fp8.gemm_scale(torch.tensor([sa], device="cuda")), dev(B), 0,
                     fp8.gemm_scale(torch.tensor([sb], device="cuda")))
        torch.cuda.synchronize()
        ref = oracle.gemm_tensor_sampled(A, "e5m2", B, "e4m3", sa, sb, ii, jj)
        t = np.float32(sa * sb)
    else:
        # per-row factors on both operands (the weight gradient's kernel), or
        # one factor per 128 rows of B (a 128x128-block weight: the wide kernel)
        KB = KMAX // 128
        gb = 1 if scaling == "block" else 128
        tA = rng.uniform(1e-6, 1e-5, (I, KB)).astype(np.float32)
        tB = rng.uniform(1e-6, 1e-5, (J // gb, KB)).astype(np.float32)
        sA, sB = oracle.BlockScale(tA, 1, KB, 1), oracle.BlockScale(tB, gb, KB, 1)
        c = fp8.gemm(dev(A), 1, fp8.gemm_scale(dev(tA), 1, KB, 1), dev(B), 0, fp8.gemm_scale(dev(tB), gb, KB, 1))
        torch.cuda.synchronize()
        ref = oracle.gemm_block_sampled(A, "e5m2", sA, B, "e4m3", sB, ii, jj)
        t = (tA, np.repeat(tB, gb, axis=0))
    got = to_np_u16(c)[ii, jj]
    print(check_gemm(got, ref, A, "e5m2", B, "e4m3", t, KMAX, "gemm K=2^23-128 " + scaling, ii, jj), flush=True)
