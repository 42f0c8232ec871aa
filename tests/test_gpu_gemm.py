"""FP8 GEMM parity on the GPU: the HIP matrix-core GEMM vs the oracle's
fp32-accumulated GEMM, within the BF16 tolerance of tests/_util.py, for every
operand-format pair the linear uses, tensorwise and block-scaled, on shapes
that span several tiles, half-full edge tiles and split-K."""
import numpy as np
import pytest
import torch

import oracle
from _util import check_bf16, mfma_window_bound, to_np_u16

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
    hw = mfma_window_bound(A, fa, B, fb, np.float32(sa * sb))
    check_bf16(to_np_u16(c), ref, K, "gemm %dx%dx%d" % (I, J, K), hw)


BLOCK_CASES = [
    # I, J, K, fa, fb, B layout ("row": 1x128 per row, "blk": 128x128, "blkT": 128x128 transposed)
    (256, 256, 512, "e4m3", "e4m3", "blk"),
    (384, 640, 256, "e4m3", "e4m3", "blk"),
    (512, 256, 512, "e5m2", "e4m3", "blkT"),
    (384, 384, 384, "e5m2", "e4m3", "row"),
    (256, 128, 16384, "e5m2", "e4m3", "row"),   # split-K
]


@pytest.mark.parametrize("I,J,K,fa,fb,bl", BLOCK_CASES)
def test_gemm_block(fp8, I, J, K, fa, fb, bl):
    rng = np.random.default_rng(I + J * 5 + K * 11)
    KB = K // 128
    A = rand_codes(fa, (I, K), rng)
    B = rand_codes(fb, (J, K), rng)
    sA_arr = rng.uniform(1e-3, 1e-1, (I, KB)).astype(np.float32)
    sA = oracle.BlockScale(sA_arr, 1, KB, 1)
    if bl == "row":
        sB_arr = rng.uniform(1e-3, 1e-1, (J, KB)).astype(np.float32)
        sB = oracle.BlockScale(sB_arr, 1, KB, 1)
        sB_full = sB_arr
    elif bl == "blk":
        sB_arr = rng.uniform(1e-3, 1e-1, (J // 128, KB)).astype(np.float32)
        sB = oracle.BlockScale(sB_arr, 128, KB, 1)
        sB_full = np.repeat(sB_arr, 128, axis=0)
    else:
        sB_arr = rng.uniform(1e-3, 1e-1, (KB, J // 128)).astype(np.float32)
        sB = oracle.BlockScale(sB_arr, 128, 1, J // 128)
        sB_full = np.repeat(sB_arr.T, 128, axis=0)
    ref = oracle.gemm_block(A, fa, sA, B, fb, sB)
    tsa, tsb = dev(sA_arr), dev(sB_arr)
    c = fp8.gemm(dev(A), FMT[fa], fp8.gemm_scale(tsa, sA.group, sA.stride_r, sA.stride_kb),
                 dev(B), FMT[fb], fp8.gemm_scale(tsb, sB.group, sB.stride_r, sB.stride_kb))
    torch.cuda.synchronize()
    hw = mfma_window_bound(A, fa, B, fb, (sA_arr, sB_full))
    check_bf16(to_np_u16(c), ref, K, "block gemm %dx%dx%d %s" % (I, J, K, bl), hw)


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
