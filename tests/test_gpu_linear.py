"""FP8 linear forward/backward on the GPU through the C ABI vs the oracle:
quantized bytes and scales bit-exact, Y / dX / dW within the BF16 tolerance;
weight cache (is_first_microbatch True/False/None) bitwise identical to
re-quantizing every microbatch; run-to-run determinism."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _util import check_gemm, to_np_u16, to_np_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_mixed_precision_amax_amd as m
    m.lib()
    return m


def cuda_bf16(t):
    return t.contiguous().cuda()


def check_q(q, ref, scaling_kind):
    """q: QTensor from the GPU; ref: oracle quantize dict."""
    assert np.array_equal(to_np_u8(q.q_row), ref["q_row"])
    assert np.array_equal(to_np_u8(q.q_col), ref["q_col"])
    f = lambda t: t.detach().cpu().numpy().view(np.uint32)
    if scaling_kind == "tensor":
        assert f(q.scale)[0] == np.float32(ref["scale"]).view(np.uint32)
        assert f(q.scale_inv)[0] == np.float32(ref["scale_inv"]).view(np.uint32)
    elif scaling_kind == "1x128":
        assert np.array_equal(f(q.scale), ref["scale_row"].view(np.uint32))
        assert np.array_equal(f(q.scale_inv), ref["scale_inv_row"].view(np.uint32))
        assert np.array_equal(f(q.scale_col), ref["scale_col"].view(np.uint32))
        assert np.array_equal(f(q.scale_inv_col), ref["scale_inv_col"].view(np.uint32))
    else:
        assert np.array_equal(f(q.scale), ref["scale"].view(np.uint32))
        assert np.array_equal(f(q.scale_inv), ref["scale_inv"].view(np.uint32))


def gemm_operands(ctx, dyq, recipe, N, K, M):
    """(name, A, fa, B, fb, t, Kc) of the three GEMMs, t as check_gemm
    takes it (scalar, or per-row / per-128-block factors of both operands)."""
    xq, wq = ctx["xq"], ctx["wq"]
    if recipe == "tensor":
        ty = np.float32(xq["scale_inv"] * wq["scale_inv"])
        tdx = np.float32(dyq["scale_inv"] * wq["scale_inv"])
        tdw = np.float32(dyq["scale_inv"] * xq["scale_inv"])
    else:
        sw = wq["scale_inv"]                                   # [M/128, K/128]
        ty = (xq["scale_inv_row"], np.repeat(sw, 128, axis=0))           # W rows m
        tdx = (dyq["scale_inv_row"], np.repeat(sw.T, 128, axis=0))       # W^T rows k
        tdw = (dyq["scale_inv_col"], xq["scale_inv_col"])
    return [("Y", xq["q_row"], "e4m3", wq["q_row"], "e4m3", ty, K),
            ("dX", dyq["q_row"], "e5m2", wq["q_col"], "e4m3", tdx, M),
            ("dW", dyq["q_col"], "e5m2", xq["q_col"], "e4m3", tdw, N)]


CASES = [
    # name, N, K, M, recipe, sigmas, outliers
    ("linear_512x512_n1024", 1024, 512, 512, "tensor", (1.0, 0.02, 1e-3), 0.0),
    ("ragged", 384, 640, 384, "tensor", (1.0, 0.02, 1e-3), 0.0),
    ("block", 1024, 512, 1024, "block", (1.0, 1.0, 1.0), 0.01),
    ("block_ragged", 640, 384, 384, "block", (1.0, 1.0, 1.0), 0.01),
]


@pytest.mark.parametrize("name,N,K,M,recipe,sig,frac", CASES)
def test_linear_parity(fp8, name, N, K, M, recipe, sig, frac):
    x, w, dy = synth.operands(N, K, M, seed=0, sigma_x=sig[0], sigma_w=sig[1], sigma_dy=sig[2], outlier_frac=frac)
    R = fp8.RECIPE_TENSOR if recipe == "tensor" else fp8.RECIPE_BLOCK
    lin = fp8.Fp8Linear(N, K, M, R)
    y = lin.forward(cuda_bf16(x), cuda_bf16(w))
    dx, dw = lin.backward(cuda_bf16(dy))
    torch.cuda.synchronize()
    yr, ctx = oracle.linear_fwd(synth.bits(x), synth.bits(w), recipe)
    dxr, dwr, dyq = oracle.linear_bwd(synth.bits(dy), ctx)
    act = "tensor" if recipe == "tensor" else "1x128"
    wsc = "tensor" if recipe == "tensor" else "128x128"
    check_q(lin.saved_x, ctx["xq"], act)
    check_q(lin.w_q, ctx["wq"], wsc)
    check_q(lin.dy_q, dyq, act)
    outs = {"Y": (y, yr), "dX": (dx, dxr), "dW": (dw, dwr)}
    for gname, A, fa, B, fb, t, Kc in gemm_operands(ctx, dyq, recipe, N, K, M):
        got, ref = outs[gname]
        print(check_gemm(to_np_u16(got), ref, A, fa, B, fb, t, Kc, name + " " + gname), flush=True)


@pytest.mark.parametrize("recipe", ["tensor", "block"])
def test_weight_cache_bitwise(fp8, recipe):
    """Gradient accumulation over 4 microbatches: cached (True, False, False,
    False) vs uncached (None x 4) give bitwise identical Y, dX, dW and
    quantized weights; the cache is filled exactly once."""
    N, K, M = 512, 512, 1024
    R = fp8.RECIPE_TENSOR if recipe == "tensor" else fp8.RECIPE_BLOCK
    g = torch.Generator().manual_seed(1000)
    w = cuda_bf16(synth.normal_bf16((M, K), 0.02, g))
    cached = fp8.Fp8Linear(N, K, M, R, cache=True)
    plain = fp8.Fp8Linear(N, K, M, R)
    for mb in range(4):
        gx = torch.Generator().manual_seed(2000 + mb)
        x = cuda_bf16(synth.normal_bf16((N, K), 1.0, gx))
        dy = cuda_bf16(synth.normal_bf16((N, M), 1e-3, gx))
        y1 = cached.forward(x, w if mb == 0 else None, is_first_microbatch=(mb == 0))
        y2 = plain.forward(x, w)
        dx1, dw1 = cached.backward(dy)
        dx2, dw2 = plain.backward(dy)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(dx1, dx2) and torch.equal(dw1, dw2), mb
        assert torch.equal(cached.weight_q().q_row, plain.weight_q().q_row)
        assert torch.equal(cached.weight_q().q_col, plain.weight_q().q_col)
        assert torch.equal(cached.weight_q().scale_inv, plain.weight_q().scale_inv)
    assert cached.cache.fills == 1 and cached.cache.valid


def test_cache_false_never_reads_weight(fp8):
    """With is_first_microbatch=False the weight pointer is not read: passing
    a different weight changes nothing."""
    N, K, M = 256, 256, 256
    x, w, _ = synth.operands(N, K, M, seed=5)
    lin = fp8.Fp8Linear(N, K, M, fp8.RECIPE_TENSOR, cache=True)
    y1 = lin.forward(cuda_bf16(x), cuda_bf16(w), is_first_microbatch=True)
    y2 = lin.forward(cuda_bf16(x), cuda_bf16(w) * 3, is_first_microbatch=False)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    lin.cache.invalidate()
    with pytest.raises(fp8.Fp8Error):
        lin.forward(cuda_bf16(x), None, is_first_microbatch=False)


def test_linear_deterministic(fp8):
    N, K, M = 2048, 512, 2048
    x, w, dy = synth.operands(N, K, M, seed=7)
    lin = fp8.Fp8Linear(N, K, M, fp8.RECIPE_TENSOR)
    outs = []
    for _ in range(2):
        y = lin.forward(cuda_bf16(x), cuda_bf16(w))
        dx, dw = lin.backward(cuda_bf16(dy))
        outs.append((y.clone(), dx.clone(), dw.clone()))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("workload", ["linear_512x2048_n131072", "linear_2048x512_n131072"])
def test_full_size_sampled(fp8, workload):
    """The two linears of the headline step (512 -> 2048 and 2048 -> 512 at
    N = 131072) in the bench's launch configuration: every quantized byte and
    scale of X, W and dY bit-exact; 4096 sampled outputs each of Y, dX and dW
    against the oracle and the matrix-core emulation."""
    print("full size", workload, flush=True)
    d = synth.workload(workload)
    N, K, M = d["N"], d["K"], d["M"]
    lin = fp8.Fp8Linear(N, K, M, fp8.RECIPE_TENSOR)
    y = lin.forward(cuda_bf16(d["x"]), cuda_bf16(d["w"]))
    dx, dw = lin.backward(cuda_bf16(d["dy"]))
    torch.cuda.synchronize()
    xq = oracle.quant_tensor(synth.bits(d["x"]), "e4m3")
    wq = oracle.quant_tensor(synth.bits(d["w"]), "e4m3")
    dyq = oracle.quant_tensor(synth.bits(d["dy"]), "e5m2")
    check_q(lin.saved_x, xq, "tensor")
    check_q(lin.w_q, wq, "tensor")
    check_q(lin.dy_q, dyq, "tensor")
    rng = np.random.default_rng(0)
    n = 4096
    for name, A, fa, sa, B, fb, sb, I, J, Kc, out in [
        ("Y", xq["q_row"], "e4m3", xq["scale_inv"], wq["q_row"], "e4m3", wq["scale_inv"], N, M, K, y),
        ("dX", dyq["q_row"], "e5m2", dyq["scale_inv"], wq["q_col"], "e4m3", wq["scale_inv"], N, K, M, dx),
        ("dW", dyq["q_col"], "e5m2", dyq["scale_inv"], xq["q_col"], "e4m3", xq["scale_inv"], M, K, N, dw),
    ]:
        ii = rng.integers(0, I, n)
        jj = rng.integers(0, J, n)
        ref = oracle.gemm_tensor_sampled(A, fa, B, fb, sa, sb, ii, jj)
        got = to_np_u16(out)[ii, jj]
        print(check_gemm(got, ref, A, fa, B, fb, np.float32(sa * sb), Kc, "full-size " + name, ii, jj), flush=True)


def test_forward_weight_larger_than_input(fp8):
    """A short microbatch against a large weight (N = 256, K = 2048,
    M = 8192): the forward quantizes X and W together with W's part of the
    launch at its workgroup cap and X's part small; both quantized tensors
    bit-exact, 2048 sampled outputs of Y against the oracle; the forward with
    the cache (W quantized alone on the second microbatch) gives the same Y."""
    N, K, M = 256, 2048, 8192
    g = torch.Generator().manual_seed(31)
    x = synth.normal_bf16((N, K), 1.0, g)
    w = synth.normal_bf16((M, K), 0.02, g)
    lin = fp8.Fp8Linear(N, K, M, fp8.RECIPE_TENSOR, cache=True)
    y = lin.forward(cuda_bf16(x), cuda_bf16(w), is_first_microbatch=True)
    y2 = lin.forward(cuda_bf16(x), None, is_first_microbatch=False)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    xq = oracle.quant_tensor(synth.bits(x), "e4m3")
    wq = oracle.quant_tensor(synth.bits(w), "e4m3")
    check_q(lin.saved_x, xq, "tensor")
    check_q(lin.weight_q(), wq, "tensor")
    rng = np.random.default_rng(3)
    ii = rng.integers(0, N, 2048)
    jj = rng.integers(0, M, 2048)
    ref = oracle.gemm_tensor_sampled(xq["q_row"], "e4m3", wq["q_row"], "e4m3", xq["scale_inv"], wq["scale_inv"], ii, jj)
    t = np.float32(xq["scale_inv"] * wq["scale_inv"])
    print(check_gemm(to_np_u16(y)[ii, jj], ref, xq["q_row"], "e4m3", wq["q_row"], "e4m3", t, K, "weight-larger Y", ii, jj),
          flush=True)
