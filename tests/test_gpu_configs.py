"""The remaining workloads at full size, through the C ABI, against the oracle.

- block scaling 512 -> 8192 at N = 131072 with 1% outliers (x100);
- the square 8192 x 8192 weight at N = 16384 and 512 -> 8192 at N = 262144,
  tensorwise and block-scaled;
(the 8-block MLP stack with the weight cache is in test_gpu_mlp_stack.py).

Every quantized byte and scale of X, W and dY is compared with the oracle
(bit-exact); Y, dX and dW are compared on 4096 sampled outputs each, to the
BF16 tolerance plus the FP8 matrix-core window bound, and to the emulation of
the matrix cores' accumulation (tests/_util.py).  Operands are drawn
with the seeded device generator (synth.workload_on_device)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _util import check_gemm_rows, to_np_u16, to_np_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_mixed_precision_amax_amd as m
    m.lib()
    return m


def _u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def check_q(q, ref, kind):
    assert np.array_equal(to_np_u8(q.q_row), ref["q_row"]), "row codes"
    assert np.array_equal(to_np_u8(q.q_col), ref["q_col"]), "col codes"
    if kind == "tensor":
        assert _u32(q.scale)[0] == np.float32(ref["scale"]).view(np.uint32)
        assert _u32(q.scale_inv)[0] == np.float32(ref["scale_inv"]).view(np.uint32)
    elif kind == "1x128":
        assert np.array_equal(_u32(q.scale), ref["scale_row"].view(np.uint32))
        assert np.array_equal(_u32(q.scale_inv), ref["scale_inv_row"].view(np.uint32))
        assert np.array_equal(_u32(q.scale_col), ref["scale_col"].view(np.uint32))
        assert np.array_equal(_u32(q.scale_inv_col), ref["scale_inv_col"].view(np.uint32))
    else:
        assert np.array_equal(_u32(q.scale), ref["scale"].view(np.uint32))
        assert np.array_equal(_u32(q.scale_inv), ref["scale_inv"].view(np.uint32))


def block_row_factors(name, q1, q2, ii, jj, N, K, M):
    """Per-row factors of every contraction block for sampled rows ii of the
    GEMM's A operand and jj of its B operand (block recipe)."""
    if name == "Y":
        return q1["scale_inv_row"][ii], q2["scale_inv"][jj // 128]
    if name == "dX":
        return q1["scale_inv_row"][ii], q2["scale_inv"].T[jj // 128]
    return q1["scale_inv_col"][ii], q2["scale_inv_col"][jj]


CONFIGS = ["linear_512x8192_n131072_block",
           "linear_8192x8192_n16384", "linear_8192x8192_n16384_block",
           "linear_512x8192_n262144", "linear_512x8192_n262144_block"]


@pytest.mark.parametrize("name", CONFIGS)
def test_config_full_size(fp8, name):
    print("config", name, flush=True)
    d = synth.workload_on_device(name, seed=0)
    N, K, M, recipe = d["N"], d["K"], d["M"], d["scaling"]
    R = fp8.RECIPE_TENSOR if recipe == "tensor" else fp8.RECIPE_BLOCK
    lin = fp8.Fp8Linear(N, K, M, R)
    y = lin.forward(d["x"], d["w"])
    dx, dw = lin.backward(d["dy"])
    torch.cuda.synchronize()
    act = "tensor" if recipe == "tensor" else "1x128"
    wsc = "tensor" if recipe == "tensor" else "128x128"
    xb, wb, dyb = synth.bits(d["x"]), synth.bits(d["w"]), synth.bits(d["dy"])
    del d
    xq = oracle.quantize(xb, "e4m3", act)
    check_q(lin.saved_x, xq, act)
    wq = oracle.quantize(wb, "e4m3", wsc)
    check_q(lin.w_q, wq, wsc)
    dyq = oracle.quantize(dyb, "e5m2", act)
    check_q(lin.dy_q, dyq, act)
    del xb, wb, dyb
    rng = np.random.default_rng(1)
    n = 4096
    for gname, (A, sA, B, sB), fa, fb, I, J, Kc, out, q1, q2 in [
        ("Y", oracle.fprop_operands(xq, wq, recipe, N, K, M), "e4m3", "e4m3", N, M, K, y, xq, wq),
        ("dX", oracle.dgrad_operands(dyq, wq, recipe, N, K, M), "e5m2", "e4m3", N, K, M, dx, dyq, wq),
        ("dW", oracle.wgrad_operands(dyq, xq, recipe, N, K, M), "e5m2", "e4m3", M, K, N, dw, dyq, xq),
    ]:
        ii = rng.integers(0, I, n)
        jj = rng.integers(0, J, n)
        if recipe == "tensor":
            ref = oracle.gemm_tensor_sampled(A, fa, B, fb, sA.s[0], sB.s[0], ii, jj)
            t = np.float32(sA.s[0] * sB.s[0])
        else:
            ref = oracle.gemm_block_sampled(A, fa, sA, B, fb, sB, ii, jj)
            t = block_row_factors(gname, q1, q2, ii, jj, N, K, M)
        got = to_np_u16(out)[ii, jj]
        rep = check_gemm_rows(got, ref, A[ii], fa, B[jj], fb, t, Kc, name + " " + gname)
        print(name, gname, rep, flush=True)
